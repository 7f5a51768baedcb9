"""Oracle-side harness for the workload configurations -- TEST INFRASTRUCTURE.

Near-tie protocol: expert ids must be compared bit-exactly, which is only
well posed when no two of the 11 largest router logits of a token lie within
a margin (1e-4 for single layers; stacks use a wider margin because the GPU's
residual stream drifts from the fp64 one by rounding).  Rows (or, for the T=1
stack, routers) that fail are redrawn from the dedicated redraw streams of
inputs.Streams.  The screen needs logits only to decide which inputs to keep,
so it uses a numpy fp64 matmul; everything compared against the GPU comes from
the oracle library.
"""
import concurrent.futures

import numpy as np

import inputs

from . import experts as _experts, route as _route, combine as _combine

TIE_MARGIN = 1e-4


def bf16_values(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rms_np(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6)


def logits_np(xhat, R_bits, bias=None):
    lg = np.asarray(xhat, dtype=np.float64) @ bf16_values(R_bits).astype(np.float64).T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float64)
    return lg


def top11_gap(lg):
    """Smallest gap between consecutive values among the 11 largest, per row."""
    s = -np.sort(-np.atleast_2d(lg), axis=1)[:, :11]
    return np.min(s[:, :-1] - s[:, 1:], axis=1)


def screened_x(st, T, R_bits, bias=None, rmsnorm=False, margin=TIE_MARGIN, h=inputs.H,
               extra=(), x_scale=1.0):
    """x [T][H] from st.x (times x_scale, in fp32); rows whose top-11 gap is
    within `margin` are redrawn from st.x_redraw, in row order.  `extra` lists
    further (router, bias) pairs the rows must also clear (a second router
    applied to the same input).  Returns (x, number of redrawn rows)."""
    x, rows = screened_x_rows(st, T, R_bits, bias, rmsnorm, margin, h, extra, x_scale)
    return x, len(rows)


def screened_x_rows(st, T, R_bits, bias=None, rmsnorm=False, margin=TIE_MARGIN, h=inputs.H,
                    extra=(), x_scale=1.0):
    """screened_x, returning the redrawn row indices in the order of their
    redraws (inputs.apply_row_redraws replays them)."""
    def draw(n, rng):
        v = inputs.draw_x(rng, n, h=h)
        return v if x_scale == 1.0 else (v * np.float32(x_scale)).astype(np.float32)
    x = draw(T, st.x)
    rows = []
    pairs = [(R_bits, bias)] + list(extra)
    for _ in range(1000):
        xh = rms_np(x) if rmsnorm else x.astype(np.float64)
        gap = np.min(np.stack([top11_gap(logits_np(xh, R, b)) for R, b in pairs]), axis=0)
        bad = np.nonzero(gap <= margin)[0]
        if bad.size == 0:
            return x, rows
        for t in bad:
            x[t] = draw(1, st.x_redraw)[0]
            rows.append(int(t))
    raise RuntimeError("near-tie screen did not converge")


def screened_windows(st, T, n, R_bits, margin=TIE_MARGIN, h=inputs.H):
    """n correlated windows [n][T][H] drawn from st.x (inputs.draw_window); a
    window with a near-tie in any token's top 11 logits is replaced by a draw
    from st.x_redraw.  Returns (windows, number of replaced windows)."""
    out, redrawn = [], 0
    for _ in range(n):
        w = inputs.draw_window(st.x, T, h=h)
        while not np.all(top11_gap(logits_np(w.astype(np.float64), R_bits, None)) > margin):
            w = inputs.draw_window(st.x_redraw, T, h=h)
            redrawn += 1
            if redrawn > 100 * n:
                raise RuntimeError("near-tie screen did not converge")
        out.append(w)
    return np.stack(out), redrawn


class BlobSource:
    """Host blobs of one seed, generated on demand (threaded) and cached."""

    def __init__(self, seed, e=inputs.E, cache=4096):
        self.seed, self.e, self.cache, self.store = seed, e, cache, {}

    def get_many(self, blob_ids):
        need = [b for b in set(int(b) for b in blob_ids) if b not in self.store]
        if need:
            with concurrent.futures.ThreadPoolExecutor(8) as ex:
                for b, arr in zip(need, ex.map(lambda b: inputs.gen_blob(self.seed, b), need)):
                    self.store[b] = arr
            if len(self.store) > self.cache:
                for b in list(self.store)[: len(self.store) - self.cache]:
                    del self.store[b]
        return {int(b): self.store[int(b)] for b in blob_ids}


def oracle_layer(x, R_bits, src, layer, bias=None, rmsnorm=False, e=inputs.E, K=inputs.K):
    """The oracle's layer on rows x (float32): returns (ids, w, y) in fp64."""
    ids, w, xhat = _route(x, R_bits, K, bias=bias, rmsnorm_flag=rmsnorm)
    got = src.get_many(layer * e + np.unique(ids))
    blobs = {b - layer * e: arr for b, arr in got.items()}
    o = _experts(xhat, ids, blobs, e, inputs.H, inputs.FF)
    return ids, w, _combine(o, w)


def stack_trajectory(x0, routers, src, biases=None, margin=TIE_MARGIN, verbose=True):
    """Run rows x0 [n][H] through len(routers) stacked layers (RMSNorm, router,
    experts, combine, residual) in the oracle.  Returns per-layer lists of ids,
    w, y, the input x of every layer, and the per-row top-11 gap per layer."""
    x = np.asarray(x0, dtype=np.float64)
    out = dict(ids=[], w=[], y=[], x_in=[], gap=[])
    for l, R in enumerate(routers):
        b = None if biases is None else biases[l]
        xf = x.astype(np.float32)
        out["gap"].append(top11_gap(logits_np(rms_np(xf), R, b)))
        ids, w, y = oracle_layer(xf, R, src, l, bias=b, rmsnorm=True)
        out["x_in"].append(xf)
        out["ids"].append(ids)
        out["w"].append(w)
        out["y"].append(y)
        x = x + y
        if verbose and (l % 8 == 7 or l == len(routers) - 1):
            print(f"  oracle trajectory: layer {l + 1}/{len(routers)} done", flush=True)
    out["x_out"] = x
    return out


def screened_stack_routers(st, x0, src, n_layers, margin, per_layer=None):
    """Routers for a T=1 stack drawn layer by layer on the oracle trajectory;
    router l is redrawn (st.router_redraw) until the row clears the margin.
    per_layer, if a list, receives the number of redraws of each layer."""
    x = np.asarray(x0, dtype=np.float64)
    routers, redraws = [], 0
    for l in range(n_layers):
        R = inputs.draw_router(st.router)
        xf = x.astype(np.float32)
        n = 0
        while top11_gap(logits_np(rms_np(xf), R))[0] <= margin:
            R = inputs.draw_router(st.router_redraw)
            redraws += 1
            n += 1
        if per_layer is not None:
            per_layer.append(n)
        routers.append(R)
        _, _, y = oracle_layer(xf, R, src, l, rmsnorm=True)
        x = x + y
        if l % 8 == 7:
            print(f"  router screen: layer {l + 1}/{n_layers} done", flush=True)
    return routers, redraws
