"""The layer with a router lookahead: its outputs are bitwise those of the
plain layer call, its predicted ids are bitwise the decode route of the same
input through the next layer's router (parity of that route with the oracle
is pinned by the route tests), and its reads of the next layer's store change
nothing."""
import numpy as np
import pytest

import harness as hz
import inputs

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


@pytest.mark.parametrize("T,flags,with_bias", [(1, 0, False), (4, 0, False), (8, 0, False),
                                               (1, 3, True), (4, 3, False), (8, 3, True)])
def test_lookahead_layer_equals_layer_and_predicts_the_next_route(T, flags, with_bias):
    import torch
    m = hz.qm()
    seed = 7000 + 10 * T + flags
    print(f"case: lookahead T={T} flags={flags} bias={with_bias}", flush=True)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, 2560)).astype(np.float32)
    R = inputs.draw_router(rng)
    R2 = inputs.draw_router(rng)
    b = inputs.draw_zipf_bias(rng) if with_bias else None
    b2 = inputs.draw_zipf_bias(rng) if with_bias else None
    st, st2 = hz.store(seed, 0), hz.store(seed, 1)
    ws = m.workspace(T)
    ids0, w0, y0, x0 = hz.gpu_layer(x, R, st, bias=b, flags=flags, ws=ws)

    xd = hz.cuda(x)
    y = torch.empty_like(xd)
    ids = torch.empty((T, 10), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 10), dtype=torch.float32, device="cuda")
    pred = torch.full((T, 10), -1, dtype=torch.int32, device="cuda")
    before = st2[:4096].clone(), st2[-4096:].clone()
    m.strata_moe_layer_lookahead(xd, hz.router_dev(R), st, ws, hz.router_dev(R2), st2,
                                 bias=None if b is None else hz.cuda(b),
                                 bias_next=None if b2 is None else hz.cuda(b2), flags=flags,
                                 y=y, ids=ids, w=w, pred=pred)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids0)
    assert np.array_equal(w.cpu().numpy(), w0)
    assert np.array_equal(y.cpu().numpy(), y0)
    assert np.array_equal(xd.cpu().numpy(), x0)   # the residual update, when asked for
    assert torch.equal(st2[:4096], before[0]) and torch.equal(st2[-4096:], before[1])

    # the prediction is the route of the same (normalised) input through R2
    pids = torch.empty((T, 10), dtype=torch.int32, device="cuda")
    pw = torch.empty((T, 10), dtype=torch.float32, device="cuda")
    m.strata_moe_route(hz.cuda(x), hz.router_dev(R2), pids, pw, m.workspace(T),
                       bias=None if b2 is None else hz.cuda(b2), flags=flags & m.RMSNORM)
    torch.cuda.synchronize()
    assert np.array_equal(pred.cpu().numpy(), pids.cpu().numpy())
    p = pred.cpu().numpy()
    assert ((p >= 0) & (p < 512)).all()
    assert all(len(set(r)) == 10 for r in p)
