"""The layer with a router lookahead ("MoE 遇上消费级显卡..." (zwxr.cn), the
passage on prefetching and warm-up: the next layer's router applied to this
layer's input predicts the next layer's experts, and warming them changes no
result).  Checked here:
 * its outputs are bitwise those of the plain layer call, and match the oracle
   layer of the same input to the parity bar;
 * its predicted ids equal the oracle's route of the same (normalised) input
   through the next layer's router and bias, as ordered lists, and are
   bitwise the decode route of that input through the C ABI;
 * its reads of the next layer's store write nothing there.
Inputs are screened for near-ties against both routers."""
import numpy as np
import pytest

import harness as hz
import inputs
import oracle
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


@pytest.mark.parametrize("T,flags,with_bias", [(1, 0, False), (2, 0, False), (4, 0, False),
                                               (8, 0, False), (1, 3, True), (3, 3, True),
                                               (4, 3, False), (8, 3, True)])
def test_lookahead_layer_equals_layer_and_predicts_the_next_route(T, flags, with_bias):
    import torch
    m = hz.qm()
    seed = 7000 + 10 * T + flags
    print(f"case: lookahead T={T} flags={flags} bias={with_bias}", flush=True)
    st_ = inputs.Streams(seed)
    R = inputs.draw_router(st_.router)
    R2 = inputs.draw_router(st_.router)
    b = inputs.draw_zipf_bias(st_.bias) if with_bias else None
    b2 = inputs.draw_zipf_bias(st_.bias) if with_bias else None
    rms = bool(flags & 1)
    x, _ = scr.screened_x(st_, T, R, bias=b, rmsnorm=rms, extra=[(R2, b2)])
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

    # the layer's own results against the oracle layer of the same input
    oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T), bias=b, rmsnorm=rms)
    hz.check(f"lookahead T={T} flags={flags} layer", ids0, w0, y0, oids, ow, oy)
    if flags & m.RESIDUAL:
        dx = np.max(np.abs(x0.astype(np.float64) - (x.astype(np.float64) + oy)))
        assert dx <= hz.Y_TOL * np.max(np.abs(oy)) + 1e-6 * np.max(np.abs(x)), dx

    # the prediction is the oracle's route of the same input through R2 (+ b2)
    p = pred.cpu().numpy()
    pids, _, _ = oracle.route(x, R2, 10, bias=b2, rmsnorm_flag=rms)
    bad = np.nonzero(np.any(p != pids, axis=1))[0]
    assert bad.size == 0, (bad, p[bad[:2]], pids[bad[:2]])

    # and bitwise the decode route of that input through the C ABI
    qids = torch.empty((T, 10), dtype=torch.int32, device="cuda")
    qw = torch.empty((T, 10), dtype=torch.float32, device="cuda")
    m.strata_moe_route(hz.cuda(x), hz.router_dev(R2), qids, qw, m.workspace(T),
                       bias=None if b2 is None else hz.cuda(b2), flags=flags & m.RMSNORM)
    torch.cuda.synchronize()
    assert np.array_equal(p, qids.cpu().numpy())


@pytest.mark.parametrize("flags,with_bias", [(0, False), (3, True)])
def test_hints_change_no_result(flags, with_bias):
    """At T = 1 the lookahead layer takes a hint (the ids the token is expected
    to route to) and requests the hinted experts' rows before its routing has
    finished.  Whatever the hint -- exact, in another order, partly wrong, with
    repeats and ids outside 0..E-1, or all wrong -- the outputs are bitwise
    those of the plain layer, and the prediction is the same."""
    import torch
    m = hz.qm()
    seed = 7300 + flags
    print(f"case: hints T=1 flags={flags} bias={with_bias}", flush=True)
    st_ = inputs.Streams(seed)
    R = inputs.draw_router(st_.router)
    R2 = inputs.draw_router(st_.router)
    b = inputs.draw_zipf_bias(st_.bias) if with_bias else None
    b2 = inputs.draw_zipf_bias(st_.bias) if with_bias else None
    rms = bool(flags & 1)
    x, _ = scr.screened_x(st_, 1, R, bias=b, rmsnorm=rms, extra=[(R2, b2)])
    st, st2 = hz.store(seed, 0), hz.store(seed, 1)
    ws = m.workspace(1)
    ids0, w0, y0, x0 = hz.gpu_layer(x, R, st, bias=b, flags=flags, ws=ws)
    others = [e for e in range(512) if e not in set(ids0[0].tolist())]
    hints = {
        "exact": ids0[0].copy(),
        "reversed": ids0[0][::-1].copy(),
        "half wrong": np.concatenate([ids0[0][:5], np.array(others[:5])]),
        "repeats and junk": np.array([ids0[0][3], ids0[0][3], -1, 512, 99999, ids0[0][0],
                                      others[0], others[0], ids0[0][9], -7]),
        "all wrong": np.array(others[10:20]),
    }
    preds = []
    for name, hv in hints.items():
        xd = hz.cuda(x)
        y = torch.empty_like(xd)
        ids = torch.empty((1, 10), dtype=torch.int32, device="cuda")
        w = torch.empty((1, 10), dtype=torch.float32, device="cuda")
        pred = torch.full((1, 10), -1, dtype=torch.int32, device="cuda")
        hint = torch.from_numpy(np.asarray(hv, dtype=np.int32).reshape(1, 10)).cuda()
        m.strata_moe_layer_lookahead(xd, hz.router_dev(R), st, ws, hz.router_dev(R2), st2,
                                     bias=None if b is None else hz.cuda(b),
                                     bias_next=None if b2 is None else hz.cuda(b2), flags=flags,
                                     y=y, ids=ids, w=w, pred=pred, hint=hint)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ids0), name
        assert np.array_equal(w.cpu().numpy(), w0), name
        assert np.array_equal(y.cpu().numpy(), y0), name
        assert np.array_equal(xd.cpu().numpy(), x0), name
        preds.append(pred.cpu().numpy())
    for p in preds[1:]:
        assert np.array_equal(p, preds[0])
    pids, _, _ = oracle.route(x, R2, 10, bias=b2, rmsnorm_flag=rms)
    assert np.array_equal(preds[0], pids)
