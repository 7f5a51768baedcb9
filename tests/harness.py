"""GPU-side helpers shared by the GPU tests (device tensors, calls through the
binding, parity checks against the oracle)."""
import numpy as np

import inputs
import oracle.screen as scr

Y_TOL = 2e-3     # max |dy| <= Y_TOL * max |y| over the compared tensor
W_TOL = 1e-5     # |dw| <= W_TOL


def qm():
    import quantized_routed_expert_router_amd as m
    return m


def cuda(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def router_dev(R_bits):
    return cuda(np.ascontiguousarray(R_bits).view(np.int16))


_stores = {}


def store(seed, layer=0):
    """Device store of one layer (cached per (seed, layer))."""
    key = (seed, layer)
    if key not in _stores:
        _stores[key] = inputs.layer_store(seed, layer)
    return _stores[key]


def drop_stores():
    _stores.clear()


def gpu_layer(x, R_bits, blobs_dev, bias=None, flags=0, ws=None):
    import torch
    m = qm()
    T = x.shape[0]
    xd = cuda(x)
    y = torch.empty_like(xd)
    ids = torch.empty((T, 10), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 10), dtype=torch.float32, device="cuda")
    ws = m.workspace(T) if ws is None else ws
    m.strata_moe_layer(xd, router_dev(R_bits), blobs_dev, ws, bias=None if bias is None else cuda(bias),
                       flags=flags, y=y, ids=ids, w=w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy(), xd.cpu().numpy()


def gpu_composed(x, R_bits, blobs_dev, bias=None, flags=0):
    """route -> group -> experts -> combine through the four entry points."""
    import torch
    m = qm()
    T = x.shape[0]
    xd = cuda(x)
    ws = m.workspace(T)
    ids = torch.empty((T, 10), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 10), dtype=torch.float32, device="cuda")
    offsets = torch.empty(513, dtype=torch.int32, device="cuda")
    slots = torch.empty(T * 10, dtype=torch.int32, device="cuda")
    active = torch.empty(513, dtype=torch.int32, device="cuda")
    out = torch.empty((T * 10, 2560), dtype=torch.float32, device="cuda")
    y = torch.empty_like(xd)
    bd = None if bias is None else cuda(bias)
    m.strata_moe_route(xd, router_dev(R_bits), ids, w, ws, bias=bd, flags=flags & m.RMSNORM)
    m.strata_moe_group(ids, offsets, slots, active, ws)
    m.strata_moe_experts(xd, blobs_dev, offsets, slots, active, out, ws, flags=flags & m.RMSNORM)
    m.strata_moe_combine(out, w, y)
    torch.cuda.synchronize()
    return dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), y=y.cpu().numpy(),
                offsets=offsets.cpu().numpy(), slots=slots.cpu().numpy(),
                active=active.cpu().numpy(), out=out.cpu().numpy())


def check(tag, ids, w, y, oids, ow, oy, w_tol=W_TOL, y_tol=Y_TOL):
    """Assert parity and return max|dy|/max|y| (all metrics printed first)."""
    assert ids.shape == oids.shape
    bad = np.nonzero(np.any(ids != oids, axis=1))[0]
    dw = float(np.max(np.abs(w.astype(np.float64) - ow)))
    ymax = float(np.max(np.abs(oy)))
    dy = np.abs(y.astype(np.float64) - oy)
    rel = float(dy.max() / ymax) if ymax > 0 else float(dy.max())
    worst_tok = float(np.max(dy.max(axis=1) / np.maximum(np.abs(oy).max(axis=1), 1e-30)))
    print(f"[{tag}] max|dy|/max|y| = {rel:.3e} (worst token {worst_tok:.3e}), max|dw| = {dw:.2e}, "
          f"rows with other ids: {bad.size}", flush=True)
    assert bad.size == 0, f"{tag}: ids differ on rows {bad[:8]}: {ids[bad[:2]]} vs {oids[bad[:2]]}"
    assert dw <= w_tol, f"{tag}: |dw| = {dw}"
    assert rel <= y_tol, f"{tag}: max|dy|/max|y| = {rel}"
    return rel


def single_layer_case(seed, T, bias=None, margin=scr.TIE_MARGIN):
    st = inputs.Streams(seed)
    R = inputs.draw_router(st.router)
    x, redrawn = scr.screened_x(st, T, R, bias=bias, margin=margin)
    return x, R, redrawn


def oracle_rows(x, R, seed, rows, bias=None, rmsnorm=False, layer=0, chunk=512, src=None):
    """The oracle's layer on rows `rows` of x, run `chunk` rows at a time (the
    per-slot expert outputs of a chunk are held in fp64).  Returns (ids, w, y)."""
    src = scr.BlobSource(seed) if src is None else src
    rows = np.asarray(rows)
    parts = []
    for i in range(0, rows.size, chunk):
        parts.append(scr.oracle_layer(x[rows[i:i + chunk]], R, src, layer, bias=bias,
                                      rmsnorm=rmsnorm))
        if rows.size > chunk:
            print(f"  oracle rows {min(i + chunk, rows.size)}/{rows.size}", flush=True)
    return tuple(np.concatenate([p[j] for p in parts]) for j in range(3))
