"""The decode experts kernel's bounded wait: when it gives up, the outputs that
depended on it are NaN and the workspace's status word says so; a normal call
leaves the word clear.  The give-up is forced from the host with a wait bound
of one poll (strata_moe_set_wait_limit), so every kernel still ends normally.
A layer call of up to three tokens runs its experts as two launches with no
wait at all (the first also routes the tokens): the bound changes nothing
there."""
import numpy as np
import pytest

import harness as hz

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hz.qm().lib()
    yield
    hz.qm().strata_moe_set_wait_limit(0)
    hz.drop_stores()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [4, 8])
def test_wait_give_up_poisons_outputs_and_sets_status(T):
    m = hz.qm()
    seed = 9100 + T
    print(f"case: forced wait give-up, layer T={T}", flush=True)
    x, R, _ = hz.single_layer_case(seed, T)
    st = hz.store(seed)
    ws = m.workspace(T)
    assert m.strata_moe_read_status(ws) == 0
    ids0, w0, y0, _ = hz.gpu_layer(x, R, st, ws=ws)
    assert m.strata_moe_read_status(ws) == 0 and np.all(np.isfinite(y0))
    m.strata_moe_set_wait_limit(1)
    try:
        ids1, w1, y1, _ = hz.gpu_layer(x, R, st, ws=ws)
    finally:
        m.strata_moe_set_wait_limit(0)
    bits = m.strata_moe_read_status(ws)
    print(f"  status {bits}, NaN rows {int(np.isnan(y1).any(axis=1).sum())}/{T}, NaN values "
          f"{int(np.isnan(y1).sum())}", flush=True)
    assert bits & m.STATUS_WAIT_TIMEOUT
    assert np.isnan(y1).any()
    assert np.array_equal(ids1, ids0) and np.array_equal(w1, w0)
    fin = ~np.isnan(y1)
    assert np.array_equal(y1[fin], y0[fin])   # what did not depend on a failed wait is exact
    # the word stays set until cleared; then a normal call leaves it clear
    ids2, w2, y2, _ = hz.gpu_layer(x, R, st, ws=ws)
    assert m.strata_moe_read_status(ws) & m.STATUS_WAIT_TIMEOUT
    m.strata_moe_clear_status(ws)
    assert m.strata_moe_read_status(ws) == 0
    ids3, w3, y3, _ = hz.gpu_layer(x, R, st, ws=ws)
    assert m.strata_moe_read_status(ws) == 0
    assert np.array_equal(y2, y0) and np.array_equal(y3, y0)


@pytest.mark.parametrize("T", [1, 3])
def test_small_layer_has_no_wait(T):
    m = hz.qm()
    seed = 9101 + T
    print(f"case: wait bound of one poll, layer T={T} (two launches)", flush=True)
    x, R, _ = hz.single_layer_case(seed, T)
    st = hz.store(seed)
    ws = m.workspace(T)
    ids0, w0, y0, _ = hz.gpu_layer(x, R, st, ws=ws)
    m.strata_moe_set_wait_limit(1)
    try:
        ids1, w1, y1, _ = hz.gpu_layer(x, R, st, ws=ws)
    finally:
        m.strata_moe_set_wait_limit(0)
    assert m.strata_moe_read_status(ws) == 0
    assert np.array_equal(ids1, ids0) and np.array_equal(w1, w0) and np.array_equal(y1, y0)
    assert np.all(np.isfinite(y1))


def test_wait_give_up_in_the_experts_entry_point():
    import torch
    m = hz.qm()
    seed, T = 9110, 3
    print("case: forced wait give-up, experts entry point T=3", flush=True)
    x, R, _ = hz.single_layer_case(seed, T)
    st = hz.store(seed)
    ref = hz.gpu_composed(x, R, st)
    ws = m.workspace(T)
    xd = hz.cuda(x)
    out = torch.empty((T * 10, 2560), dtype=torch.float32, device="cuda")
    args = [hz.cuda(ref[k]) for k in ("offsets", "slots", "active")]
    m.strata_moe_set_wait_limit(1)
    try:
        m.strata_moe_experts(xd, st, *args, out, ws)
    finally:
        m.strata_moe_set_wait_limit(0)
    o = out.cpu().numpy()
    assert m.strata_moe_read_status(ws) & m.STATUS_WAIT_TIMEOUT
    assert np.isnan(o).any()
    fin = ~np.isnan(o)
    assert np.array_equal(o[fin], ref["out"][fin])
