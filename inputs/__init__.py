"""Seeded synthetic inputs for the routed-expert MoE layer.

This module is shared by the tests, the oracle harness and bench.py.  It holds
none of the layer's arithmetic (no decode, no router, no softmax, no expert):
it only draws numbers and encodes them into the formats the layer consumes.

Expert blobs come from a counter-based generator so that the host (this file,
numpy) and the device (inputs/fill.hip) produce identical bytes for any
(seed, blob id) without transferring 34 GB:

  SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; constants of Vigna's splitmix64.c):
      mix(z)  = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
                z ^= z >> 27; z *= 0x94D049BB133111EB; z ^ (z >> 31)
      out(state, i) = mix(state + (i + 1) * 0x9E3779B97F4A7C15)   (i >= 0)

  blob key    k(seed, b) = out(out(seed, 0), b),  b = layer * E + expert
  blob word   W(seed, b, i) = out(k(seed, b), i)
  block n of a blob (byte offset 18 n, gate then up then down):
      bytes 2..9   = little-endian W(3n),  bytes 10..17 = little-endian W(3n+1)
      bytes 0..1   = SCALE_TABLE[W(3n+2) >> 48]   (little-endian fp16)

SCALE_TABLE[i] = fp16_rne(0.01 * Q((i + 0.5) / 65536) + 1e-4), Q the half-normal
quantile, i.e. a 16-bit inverse-CDF draw of |N(0, 0.01)| + 1e-4 (the scale law
of the workload); the table is computed here once and handed to the device.

x, routers and Zipf biases use numpy's PCG64 streams spawned from
SeedSequence(seed): [x, routers, bias, x redraws, router redraws].
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

# Layer geometry of the workload (48 layers x 512 experts, top-10, H=2560, FF=640).
H, FF, E, K, L = 2560, 640, 512, 10, 48
QK, BB = 64, 18


def _mix(z):
    z = (z ^ (z >> np.uint64(30))) * M1
    z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def splitmix64(state, idx):
    """Outputs number idx (array, 0-based) of the SplitMix64 stream at `state`."""
    with np.errstate(over="ignore"):
        st = np.uint64(state)
        i = np.asarray(idx, dtype=np.uint64)
        return _mix(st + (i + np.uint64(1)) * GAMMA)


def blob_key(seed, blob_id):
    base = splitmix64(np.uint64(seed), np.array([0], dtype=np.uint64))[0]
    return splitmix64(base, np.array([blob_id], dtype=np.uint64))[0]


_TABLE = None


def scale_table():
    """uint16[65536] fp16 bit patterns of the scale law (see module doc)."""
    global _TABLE
    if _TABLE is None:
        from scipy.special import ndtri
        u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        z = ndtri(0.5 + 0.5 * u)  # half-normal quantile
        _TABLE = (0.01 * z + 1e-4).astype(np.float16).view(np.uint16).copy()
    return _TABLE


def blob_bytes(h=H, ff=FF):
    return 3 * (h * ff * BB // QK)


def gen_blob(seed, blob_id, h=H, ff=FF):
    """The bytes of blob `blob_id` (= layer * E + expert) as uint8[blob_bytes]."""
    nblk = 3 * h * ff // QK
    key = blob_key(seed, blob_id)
    n = np.arange(nblk, dtype=np.uint64)
    w0 = splitmix64(key, np.uint64(3) * n)
    w1 = splitmix64(key, np.uint64(3) * n + np.uint64(1))
    w2 = splitmix64(key, np.uint64(3) * n + np.uint64(2))
    out = np.empty((nblk, BB), dtype=np.uint8)
    sc = scale_table()[(w2 >> np.uint64(48)).astype(np.int64)]
    out[:, 0:2] = sc.astype("<u2").view(np.uint8).reshape(nblk, 2)
    out[:, 2:10] = w0.astype("<u8").view(np.uint8).reshape(nblk, 8)
    out[:, 10:18] = w1.astype("<u8").view(np.uint8).reshape(nblk, 8)
    return out.reshape(-1)


def f32_to_bf16_bits(a):
    """Round-to-nearest-even of float32 values to bfloat16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


class Streams:
    """The five numpy streams of one seed, in the fixed spawn order."""

    def __init__(self, seed):
        ch = np.random.SeedSequence(seed).spawn(5)
        self.x, self.router, self.bias, self.x_redraw, self.router_redraw = (
            np.random.Generator(np.random.PCG64(c)) for c in ch)


def draw_x(rng, T, h=H):
    return rng.standard_normal((T, h)).astype(np.float32)


# Correlated verify windows: token t of a window of T tokens is
# x_t = c u + sqrt(1 - c^2) z_t with u, z_t ~ N(0, I) (so every x_t is N(0, I)
# like the other workloads' tokens).  c per window size was chosen by
# simulation with the router recipe below and top-10 routing so that a
# window's distinct experts average 1.75, 2.4 and 3.05 times one token's 10
# for T = 2, 3, 4 -- the multiples "Strata in the source..." quotes in "The
# plan: three destinations per expert".
WINDOW_CORR = {2: 0.79, 3: 0.78, 4: 0.75}


def draw_window(rng, T, h=H):
    c = WINDOW_CORR[T]
    u = rng.standard_normal(h)
    z = rng.standard_normal((T, h))
    return (c * u[None, :] + np.sqrt(1.0 - c * c) * z).astype(np.float32)


def draw_router(rng, e=E, h=H):
    """bf16(N(0, 0.02)) router [E][H] as uint16 bit patterns."""
    return f32_to_bf16_bits((rng.standard_normal((e, h)) * 0.02).astype(np.float32))


def draw_zipf_bias(rng, e=E, s=1.1):
    """b_e = -s * ln(rank_e), rank = a seeded permutation of 1..E (fp32)."""
    rank = rng.permutation(e).astype(np.float64) + 1.0
    return (-s * np.log(rank)).astype(np.float32)


# The five workload configurations: tokens, layers, seed, stack flags.
_WORKLOAD_LIST = [
    dict(name="layer-T1", T=1, layers=1, seed=0, stack=False, zipf=False, chunk=1),
    dict(name="layer-T4-window", T=4, layers=1, seed=1, stack=False, zipf=False, chunk=4),
    dict(name="stack48-T1", T=1, layers=48, seed=2, stack=True, zipf=False, chunk=1),
    dict(name="layer-T2048-prefill", T=2048, layers=1, seed=3, stack=False, zipf=False,
         chunk=2048),
    dict(name="stack48-T32768-zipf", T=32768, layers=48, seed=4, stack=True, zipf=True,
         chunk=2048),
    # a T = 4 verify window of correlated tokens (draw_window), for the
    # window-dedup workload
    dict(name="layer-T4-correlated-window", T=4, layers=1, seed=5, stack=False, zipf=False,
         chunk=4, window=True),
]
# The seeded synthetic workloads, by name.
WORKLOADS = {w["name"]: w for w in _WORKLOAD_LIST}


# ---------------------------------------------------------------- device side
_fill_lib = None
_tables = {}


def _fill_library():
    global _fill_lib
    if _fill_lib is None:
        import ctypes
        import os
        from . import build as _b
        if not os.path.exists(_b.LIB):
            raise RuntimeError(f"{_b.LIB} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(_b.LIB)
        L.strata_inputs_fill_blobs.restype = ctypes.c_int
        L.strata_inputs_fill_blobs.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_void_p, ctypes.c_void_p]
        _fill_lib = L
    return _fill_lib


def fill_blobs_device(dst, seed, first_blob, n_blobs, h=H, ff=FF, stream=None):
    """Write blobs first_blob .. first_blob+n_blobs-1 of `seed` into the uint8
    CUDA tensor dst (at its start), byte-identical to gen_blob()."""
    import torch
    need = n_blobs * blob_bytes(h, ff)
    if dst.numel() < need or dst.dtype != torch.uint8 or not dst.is_cuda:
        raise ValueError("destination too small or not a uint8 GPU tensor")
    key = str(dst.device)
    if key not in _tables:
        _tables[key] = torch.from_numpy(scale_table().view(np.int16).copy()).to(dst.device)
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = _fill_library().strata_inputs_fill_blobs(dst.data_ptr(), int(seed), int(first_blob),
                                                  int(n_blobs), h, ff, _tables[key].data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"strata_inputs_fill_blobs failed with {rc}")


def layer_store(seed, layer, device="cuda", n_layers=1, e=E):
    """A device tensor holding n_layers consecutive layer stores (layer-major,
    e blobs each) starting at `layer`, generated on the device."""
    import torch
    store = torch.empty(n_layers * e * blob_bytes(), dtype=torch.uint8, device=device)
    fill_blobs_device(store, seed, layer * e, n_layers * e)
    return store


# ---------------------------------------------------------------- screened workloads
def apply_row_redraws(st, x, rows, h=H):
    """Replace rows of x, in the listed order, by fresh draws from st.x_redraw
    (the replay of a near-tie screen's decisions)."""
    for t in rows:
        x[t] = draw_x(st.x_redraw, 1, h=h)[0]
    return x


def _screens():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "screens.json")
    with open(path) as f:
        return json.load(f)


def workload_inputs(name, T=None):
    """x, the routers and the biases of a workload configuration, with the
    stored near-tie screen decisions replayed (screens.json, written by
    oracle/write_screens.py): the inputs the parity tests check.  T overrides
    the token count of the unscreened Zipf stack only (one chunk of it)."""
    c = WORKLOADS[name]
    st = Streams(c["seed"])
    scr = _screens().get(name, {})
    routers, biases = [], None
    if c.get("window"):
        x = draw_window(st.x, c["T"])
        routers = [draw_router(st.router)]
        for _ in range(scr.get("window_redraws", 0)):
            x = draw_window(st.x_redraw, c["T"])
    elif name == "stack48-T1":
        x = draw_x(st.x, 1)
        for n in scr["router_redraws"]:
            R = draw_router(st.router)
            for _ in range(n):
                R = draw_router(st.router_redraw)
            routers.append(R)
    elif name == "stack48-T32768-zipf":
        x = draw_x(st.x, c["T"] if T is None else T)
        routers = [draw_router(st.router) for _ in range(c["layers"])]
        biases = [draw_zipf_bias(st.bias) for _ in range(c["layers"])]
    else:
        routers = [draw_router(st.router)]
        x = apply_row_redraws(st, draw_x(st.x, c["T"]), scr["x_redraw_rows"])
    return x, routers, biases
