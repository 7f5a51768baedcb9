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
   prefill stack (32,768 Zipf-routed tokens; the per-layer check runs on 4
   seeded layers x 64 seeded tokens) the residual stream grows to |x| ~ 1e2
   within a few layers and a token's experts can change with that drift, so
   the end-to-end part checks properties of the GPU's own results (row
   weights sum to 1, distinct ids, final x = x0 + the layers' y), the first
   layer against the oracle at the full bar, and bounds the drift from the
   oracle trajectories on the rows still on the oracle's experts.
"""
import numpy as np
import pytest

import harness as hz
import inputs
import oracle.screen as scr

pytestmark = pytest.mark.gpu

# The GPU's fp32 residual stream drifts from the fp64 one by rounding over 48
# layers, so the T=1 stack keeps a wider router margin than single layers
# (the margin is also the one of the stored screen decisions that bench.py
# replays).
from oracle.write_screens import STACK_MARGIN_T1  # noqa: E402

# End-to-end drift bounds, about twice the drift measured on MI355X (T=1
# stack: max|dw| 5.4e-6 over 48 layers; Zipf stack: max|dy|/max|y| 2.6e-2 and
# max|dw| 2.5e-2 on the rows still on the oracle's experts).  The per-layer
# checks on identical inputs hold the full single-layer bar.
W_TOL_STACK = 1.1e-5
ZIPF_E2E_DY = 5e-2
ZIPF_E2E_DW = 5e-2


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
    worst, worst_dw = 0.0, 0.0
    for l in range(48):
        worst = max(worst, hz.check(f"stack48-T1 e2e layer {l}", got["ids"][l], got["w"][l],
                                    got["y"][l], traj["ids"][l], traj["w"][l], traj["y"][l],
                                    w_tol=W_TOL_STACK))
        worst_dw = max(worst_dw, float(np.max(np.abs(got["w"][l] - traj["w"][l]))))
    dx = np.max(np.abs(got["x"] - traj["x_out"])) / np.max(np.abs(traj["x_out"]))
    print(f"stack48-T1: worst end-to-end layer max|dy|/max|y| {worst:.3e}, max|dw| "
          f"{worst_dw:.2e}, final x {dx:.3e}", flush=True)
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


N_SAMPLED_LAYERS = 4
N_SAMPLED_TOKENS = 64


@pytest.mark.timeout(1800)
def test_stack48_t32768_zipf_sampled():
    """The 32,768-token Zipf stack (16 chunks of 2048 through 48 layers).

    Sample: 4 seeded layers and 64 seeded tokens.  Candidate tokens are taken
    in a seeded order; the oracle runs each candidate's whole trajectory, and a
    candidate is kept if its router input clears the 1e-4 near-tie margin at
    all 4 sampled layers, else it is excluded (and reported) and the next
    candidate is taken, until 64 are kept.  Per sampled layer, the GPU layer
    runs on the oracle's own layer input of the 64 tokens, placed inside a
    full 2048-token chunk, and must meet the single-layer bar on those rows.
    End to end, the GPU stack runs on its own residual stream; its drift from
    the oracle trajectories is measured and bounded."""
    c = inputs.WORKLOADS["stack48-T32768-zipf"]
    seed, T, chunk = c["seed"], c["T"], c["chunk"]
    st = inputs.Streams(seed)
    x = inputs.draw_x(st.x, T)
    routers = [inputs.draw_router(st.router) for _ in range(48)]
    biases = [inputs.draw_zipf_bias(st.bias) for _ in range(48)]
    pick = np.random.default_rng(44)
    layers = np.sort(pick.choice(48, N_SAMPLED_LAYERS, replace=False))
    order = pick.permutation(T)
    src = scr.BlobSource(seed, cache=30000)
    print(f"case: stack48-T32768-zipf sampled layers {list(layers)}; oracle trajectories",
          flush=True)
    kept, excluded, trajs = [], [], []
    pos = 0
    while len(kept) < N_SAMPLED_TOKENS:
        need = N_SAMPLED_TOKENS - len(kept)
        cand = order[pos:pos + need + max(4, need // 8)]
        pos += cand.size
        tr = scr.stack_trajectory(x[cand], routers, src, biases)
        gaps = np.min(np.stack([tr["gap"][l] for l in layers]), axis=0)
        for i, tok in enumerate(cand):
            if gaps[i] > scr.TIE_MARGIN and len(kept) < N_SAMPLED_TOKENS:
                kept.append(int(tok))
                trajs.append((tr, i))
            elif gaps[i] <= scr.TIE_MARGIN:
                excluded.append(int(tok))
    print(f"stack48-T32768-zipf: {len(kept)} tokens kept, {len(excluded)} excluded for a near-tie "
          f"at a sampled layer: {excluded}", flush=True)

    def traj(key, l):
        return np.stack([tr[key][l][i] for tr, i in trajs])

    store = inputs.layer_store(seed, 0, n_layers=48)
    per = 512 * inputs.blob_bytes()
    # per sampled layer, on the oracle's own inputs inside a full chunk
    for l in layers:
        xin = x[:chunk].copy()
        xin[:N_SAMPLED_TOKENS] = traj("x_in", l)
        ids, w, y, _ = hz.gpu_layer(xin, routers[l], store[l * per:(l + 1) * per],
                                    bias=biases[l], flags=3)
        n = N_SAMPLED_TOKENS
        hz.check(f"stack48-T32768-zipf sampled layer {l}", ids[:n], w[:n], y[:n],
                 traj("ids", l), traj("w", l), traj("y", l))

    # end to end on the GPU's own residual stream
    print("case: stack48-T32768-zipf GPU, 16 chunks x 48 layers", flush=True)
    kept_a = np.array(kept)
    got = {k: [[None] * len(kept) for _ in range(48)] for k in ("ids", "w", "y")}
    gx = [None] * len(kept)
    for ch in range(T // chunk):
        lo, hi = ch * chunk, (ch + 1) * chunk
        sel = np.nonzero((kept_a >= lo) & (kept_a < hi))[0]
        if sel.size == 0:
            continue
        r = _run_stack_gpu(x[lo:hi], routers, store, biases, rows=kept_a[sel] - lo)
        for j, i in enumerate(sel):
            for k in ("ids", "w", "y"):
                for l in range(48):
                    got[k][l][i] = r[k][l][j]
            gx[i] = r["x"][j]
    got = {k: [np.stack(v) for v in got[k]] for k in got}
    gx = np.stack(gx)
    xs = x[kept_a].astype(np.float32)
    worst_dy, worst_dw, rows_off = 0.0, 0.0, 0
    for l in range(48):
        gi, gw, gy = got["ids"][l], got["w"][l], got["y"][l]
        assert np.all((gi >= 0) & (gi < 512)), l
        assert all(len(set(r)) == 10 for r in gi), l
        assert np.max(np.abs(gw.astype(np.float64).sum(axis=1) - 1.0)) <= hz.W_TOL, l
        assert np.all(np.isfinite(gy)), l
        oi, ow, oy = traj("ids", l), traj("w", l), traj("y", l)
        if l == 0:   # the first layer sees identical inputs: the full bar
            hz.check("stack48-T32768-zipf e2e layer 0", gi, gw, gy, oi, ow, oy)
        same = np.all(gi == oi, axis=1)
        rows_off = max(rows_off, int((~same).sum()))
        on = np.nonzero(same)[0]
        if on.size:
            dy = float(np.max(np.abs(gy[on] - oy[on])) / np.max(np.abs(oy[on])))
            dw = float(np.max(np.abs(gw[on] - ow[on])))
            worst_dy, worst_dw = max(worst_dy, dy), max(worst_dw, dw)
        print(f"[stack48-T32768-zipf e2e layer {l}] rows on the oracle trajectory's experts "
              f"{int(same.sum())}/{len(kept)}, drift on them max|dy|/max|y| "
              f"{dy if on.size else 0.0:.3e} max|dw| {dw if on.size else 0.0:.2e}", flush=True)
        xs = (xs + gy.astype(np.float32)).astype(np.float32)
    print(f"stack48-T32768-zipf e2e: worst drift max|dy|/max|y| {worst_dy:.3e}, max|dw| "
          f"{worst_dw:.2e}, most rows off the oracle's experts at one layer {rows_off}",
          flush=True)
    assert worst_dy <= ZIPF_E2E_DY and worst_dw <= ZIPF_E2E_DW, (worst_dy, worst_dw)
    assert np.array_equal(xs, gx)   # the residual stream is x0 plus the layers' y
