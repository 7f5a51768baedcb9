"""48-layer stacks (RMSNorm -> router -> experts -> combine -> residual) at
the workload's full sizes, compared with full oracle trajectories of the same
tokens.  The oracle only ever sees generator inputs.

Two checks per stack:
 * per layer, on identical inputs: the GPU layer l is run on the oracle's own
   layer-l input (uploaded), and must meet the single-layer bar (ids exact,
   |dw| <= 1e-5, max|dy| <= 2e-3 max|y|);
 * end to end: the GPU stack runs on its own residual stream.  For the T=1
   decode stack (routers screened with a wide margin) ids must match the
   oracle trajectory at every layer and y, x stay within 2e-3 of max|.|; w
   inherits the fp32 residual drift, so it only gets W_TOL_STACK.  For the
   prefill stack the residual stream grows to |x| ~ 1e2 within a few layers
   and a token's experts can change with that drift, so the end-to-end part
   there checks properties of the GPU's own results (row weights sum to 1,
   distinct ids, final x = x0 + the layers' y), the first layer against the
   oracle, and reports the drift from the oracle trajectory.
"""
import numpy as np
import pytest

import harness as hz
import inputs
import oracle.screen as scr

pytestmark = pytest.mark.gpu

# The GPU's fp32 residual stream drifts from the fp64 one by rounding over 48
# layers, so stacked runs keep a wider router margin than single layers.
STACK_MARGIN_T1 = 1e-3
STACK_MARGIN_PREFILL = 3e-4
W_TOL_STACK = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hz.qm().lib()
    yield
    hz.drop_stores()
    torch.cuda.empty_cache()


def _run_stack_gpu(x, routers, store, biases=None, rows=None):
    """All layers on the GPU for x [T][H]; returns per-layer ids, w, y of `rows`."""
    import torch
    m = hz.qm()
    T = x.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    ridx = torch.from_numpy(rows).cuda()
    xd = hz.cuda(x)
    ws = m.workspace(T)
    y = torch.empty_like(xd)
    ids = torch.empty((T, 10), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 10), device="cuda")
    got = dict(ids=[], w=[], y=[])
    Rd = [hz.router_dev(R) for R in routers]
    bd = None if biases is None else [hz.cuda(b) for b in biases]
    per = 512 * inputs.blob_bytes()
    for l in range(len(routers)):
        m.strata_moe_layer(xd, Rd[l], store[l * per:(l + 1) * per], ws,
                           bias=None if bd is None else bd[l], flags=m.RMSNORM | m.RESIDUAL,
                           y=y, ids=ids, w=w)
        got["ids"].append(ids.index_select(0, ridx).cpu().numpy())
        got["w"].append(w.index_select(0, ridx).cpu().numpy())
        got["y"].append(y.index_select(0, ridx).cpu().numpy())
    got["x"] = xd.index_select(0, ridx).cpu().numpy()
    return got


@pytest.mark.timeout(900)
def test_stack48_t1():
    c = inputs.WORKLOADS["stack48-T1"]
    seed = c["seed"]
    st = inputs.Streams(seed)
    x0 = inputs.draw_x(st.x, 1)
    src = scr.BlobSource(seed)
    print("case: stack48-T1 screening routers on the oracle trajectory", flush=True)
    routers, redraws = scr.screened_stack_routers(st, x0, src, 48, STACK_MARGIN_T1)
    traj = scr.stack_trajectory(x0, routers, src)
    print(f"stack48-T1: {redraws} router redraws; min gap {min(g.min() for g in traj['gap']):.2e}",
          flush=True)
    store = inputs.layer_store(seed, 0, n_layers=48)
    print("case: stack48-T1 GPU stack (48 layers, 34 GB store)", flush=True)
    got = _run_stack_gpu(x0, routers, store)
    worst = 0.0
    for l in range(48):
        worst = max(worst, hz.check(f"stack48-T1 e2e layer {l}", got["ids"][l], got["w"][l],
                                    got["y"][l], traj["ids"][l], traj["w"][l], traj["y"][l],
                                    w_tol=W_TOL_STACK))
    dx = np.max(np.abs(got["x"] - traj["x_out"])) / np.max(np.abs(traj["x_out"]))
    print(f"stack48-T1: worst end-to-end layer {worst:.3e}, final x {dx:.3e}", flush=True)
    assert dx <= hz.Y_TOL
    # the byte budget: 48 x 10 distinct blobs were read for the token
    assert sum(len(set(i.ravel())) for i in got["ids"]) == 480
    # per layer on the oracle's own inputs: the single-layer bar
    per = 512 * inputs.blob_bytes()
    for l in range(48):
        ids, w, y, xo = hz.gpu_layer(traj["x_in"][l], routers[l], store[l * per:(l + 1) * per],
                                     flags=3)
        hz.check(f"stack48-T1 forced layer {l}", ids, w, y, traj["ids"][l], traj["w"][l],
                 traj["y"][l])


@pytest.mark.timeout(1200)
def test_stack48_t32768_zipf_sampled():
    c = inputs.WORKLOADS["stack48-T32768-zipf"]
    seed, T, chunk = c["seed"], c["T"], c["chunk"]
    st = inputs.Streams(seed)
    x = inputs.draw_x(st.x, T)
    routers = [inputs.draw_router(st.router) for _ in range(48)]
    biases = [inputs.draw_zipf_bias(st.bias) for _ in range(48)]
    cand = np.sort(np.random.default_rng(44).choice(T, 24, replace=False))
    store = inputs.layer_store(seed, 0, n_layers=48)
    print("case: stack48-T32768-zipf GPU, 16 chunks x 48 layers", flush=True)
    got = {k: [[] for _ in range(48)] for k in ("ids", "w", "y")}
    gx = []
    for ch in range(T // chunk):
        lo, hi = ch * chunk, (ch + 1) * chunk
        rows = cand[(cand >= lo) & (cand < hi)] - lo
        r = _run_stack_gpu(x[lo:hi], routers, store, biases, rows=rows)
        for k in ("ids", "w", "y"):
            for l in range(48):
                got[k][l].append(r[k][l])
        gx.append(r["x"])
    for k in ("ids", "w", "y"):
        got[k] = [np.concatenate(v) for v in got[k]]
    gx = np.concatenate(gx)
    print("case: stack48-T32768-zipf oracle trajectories of 24 sampled tokens", flush=True)
    src = scr.BlobSource(seed, cache=20000)
    traj = scr.stack_trajectory(x[cand], routers, src, biases)
    gaps = np.min(np.stack(traj["gap"]), axis=0)
    keep = np.nonzero(gaps > STACK_MARGIN_PREFILL)[0]
    print(f"stack48-T32768-zipf: {keep.size}/24 tokens clear the {STACK_MARGIN_PREFILL} margin at all 48 "
          f"layers", flush=True)
    assert keep.size >= 6
    # per layer on the oracle's own inputs, inside a full 2048-token chunk (so
    # the prefill kernels run as in the stack); the other rows are chunk 0's
    # generator rows
    per = 512 * inputs.blob_bytes()
    k = keep.size
    for l in range(48):
        xin = x[:chunk].copy()
        xin[:k] = traj["x_in"][l][keep]
        ids, w, y, _ = hz.gpu_layer(xin, routers[l], store[l * per:(l + 1) * per],
                                    bias=biases[l], flags=3)
        hz.check(f"stack48-T32768-zipf forced layer {l}", ids[:k], w[:k], y[:k], traj["ids"][l][keep],
                 traj["w"][l][keep], traj["y"][l][keep])
    # end to end on the GPU's own residual stream.  The fp32 stream drifts from
    # the fp64 trajectory (this stack's residual grows to |x| ~ 1e2), so after
    # some layers a token may legitimately take other experts; the strict bar
    # is the per-layer check above.  Here: properties of the GPU's own results
    # (weights of a row sum to 1, ids distinct and in range, the final x is x0
    # plus the layers' y in fp32), the first layer equal to the oracle's, and
    # the drift from the oracle trajectory reported (bounded grossly while a
    # token is still on the oracle's experts).
    xs = x[cand].astype(np.float32)
    for l in range(48):
        gi, gw, gy = got["ids"][l], got["w"][l], got["y"][l]
        assert np.all((gi >= 0) & (gi < 512)), l
        assert all(len(set(r)) == 10 for r in gi), l
        assert np.max(np.abs(gw.astype(np.float64).sum(axis=1) - 1.0)) <= hz.W_TOL, l
        assert np.all(np.isfinite(gy)), l
        same = np.all(gi == traj["ids"][l], axis=1)
        if l == 0:
            hz.check("stack48-T32768-zipf e2e layer 0", gi[keep], gw[keep], gy[keep], traj["ids"][0][keep],
                     traj["w"][0][keep], traj["y"][0][keep])
        on = keep[same[keep]]
        dy = (float(np.max(np.abs(gy[on] - traj["y"][l][on])) / np.max(np.abs(traj["y"][l][on])))
              if on.size else 0.0)
        print(f"[stack48-T32768-zipf e2e layer {l}] rows on the oracle trajectory's experts "
              f"{int(same.sum())}/{len(cand)}, drift max|dy|/max|y| on them {dy:.3e}", flush=True)
        assert dy <= 0.1, (l, dy)
        xs = (xs + gy.astype(np.float32)).astype(np.float32)
    assert np.array_equal(xs, gx)   # the residual stream is x0 plus the layers' y
