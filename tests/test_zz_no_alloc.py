"""strata_moe_layer_static -- the layer without a workspace argument, for
callers that cannot allocate -- against strata_moe_layer: calls in a row, each
with fewer tokens than the one before (the prefill path at the static limit
of 64 tokens, then 20, then the decode path at 16, 4 and 1), each bitwise
equal to the workspace call (ids, w, y and the residual update) and within
the oracle's parity bar."""
import numpy as np
import pytest

import harness as hz
import inputs
import oracle.screen as scr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hz.qm().lib()
    yield
    hz.drop_stores()
    torch.cuda.empty_cache()


def test_static_layer_matches_the_workspace_layer_on_shrinking_calls():
    import torch
    m = hz.qm()
    seed = 9200
    store = hz.store(seed)
    for i, (T, flags) in enumerate([(64, 0), (20, 3), (16, 0), (4, 3), (1, 0)]):
        print(f"case: static-workspace layer call {i}: T={T} flags={flags}", flush=True)
        st = inputs.Streams(seed + T)
        R = inputs.draw_router(st.router)
        x, _ = scr.screened_x(st, T, R, rmsnorm=bool(flags & 1))
        ids0, w0, y0, x0 = hz.gpu_layer(x, R, store, flags=flags)
        xd = hz.cuda(x)
        y = torch.full_like(xd, float("nan"))
        ids = torch.full((T, 10), -1, dtype=torch.int32, device="cuda")
        w = torch.full((T, 10), float("nan"), dtype=torch.float32, device="cuda")
        m.strata_moe_layer_static(xd, hz.router_dev(R), store, flags=flags, y=y, ids=ids, w=w)
        torch.cuda.synchronize()
        ids1, w1, y1, x1 = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy(), xd.cpu().numpy()
        assert np.array_equal(ids1, ids0) and np.array_equal(w1, w0), i
        assert np.array_equal(y1, y0) and np.array_equal(x1, x0), i
        oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T), rmsnorm=bool(flags & 1))
        hz.check(f"static layer T={T}", ids1, w1, y1, oids, ow, oy)


def test_static_layer_refuses_more_tokens_than_its_workspace_holds():
    import torch
    m = hz.qm()
    x = torch.zeros((65, 2560), device="cuda")
    R = torch.zeros((512, 2560), dtype=torch.int16, device="cuda")
    L = m.lib()
    rc = L.strata_moe_layer_static(x.data_ptr(), 65, R.data_ptr(), None, 0x10000, 0,
                                   x.data_ptr(), None, None, None)
    assert rc == m.E_SHAPE
