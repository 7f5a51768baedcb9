"""CPU oracle of the routed-expert MoE layer -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  It wraps oracle/libstrata_oracle.so (plain fp64 C, see
strata_oracle.c for the readings it follows) with numpy marshalling only.
"""
import contextlib
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)

RENORM_CLAMP = 2.0 ** -14  # the reading of "ggml's lower clamp"; provably inactive
RMS_EPS = 1e-6


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = _load(_build.LIB)
    return _lib


@contextlib.contextmanager
def using(path):
    """Temporarily route every call to another build of the oracle source
    (used by the tests that plant mistakes in a copy of it)."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def _load(path):
    L = ctypes.CDLL(path)
    L.orc_blob_bytes.restype = ctypes.c_size_t
    L.orc_blob_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    L.orc_half_to_double.restype = ctypes.c_double
    L.orc_half_to_double.argtypes = [ctypes.c_uint16]
    L.orc_bf16_to_double.restype = ctypes.c_double
    L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    L.orc_q2_code.restype = ctypes.c_int
    L.orc_q2_code.argtypes = [_u8p, ctypes.c_int]
    L.orc_q2_value.restype = ctypes.c_double
    L.orc_q2_value.argtypes = [_u8p, ctypes.c_int]
    L.orc_decode_matrix.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, _f64p]
    L.orc_rmsnorm.argtypes = [_f64p, ctypes.c_int, ctypes.c_double, _f64p]
    L.orc_silu.restype = ctypes.c_double
    L.orc_silu.argtypes = [ctypes.c_double]
    L.orc_router_logits.argtypes = [_f64p, _u16p, _f32p, ctypes.c_int, ctypes.c_int, _f64p]
    L.orc_softmax_topk.argtypes = [_f64p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                   _i32p, _f64p, _f64p]
    L.orc_expert.argtypes = [_u8p, _f64p, ctypes.c_int, ctypes.c_int, _f64p]
    L.orc_route.argtypes = [ctypes.c_int] * 4 + [_f32p, ctypes.c_int, ctypes.c_double, _u16p,
                                                 _f32p, ctypes.c_double, _i32p, _f64p, _f64p]
    L.orc_experts.argtypes = [ctypes.c_int] * 5 + [_f64p, _i32p,
                                                   ctypes.POINTER(ctypes.c_void_p), _f64p]
    L.orc_combine.argtypes = [ctypes.c_int] * 3 + [_f64p, _f64p, _f64p]
    L.orc_num_threads.restype = ctypes.c_int
    return L


def _p(a, t):
    return a.ctypes.data_as(t)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with {rc}")


def blob_bytes(H, FF):
    return int(lib().orc_blob_bytes(H, FF))


def half_to_double(h):
    return lib().orc_half_to_double(int(h))


def bf16_to_double(b):
    return lib().orc_bf16_to_double(int(b))


def q2_codes(block):
    blk = np.ascontiguousarray(np.frombuffer(bytes(block), dtype=np.uint8))
    return [lib().orc_q2_code(_p(blk, _u8p), i) for i in range(64)]


def decode_matrix(mat, rows, cols):
    if not isinstance(mat, np.ndarray):
        mat = np.frombuffer(bytes(mat), dtype=np.uint8)
    mat = np.ascontiguousarray(mat, dtype=np.uint8)
    w = np.empty((rows, cols), dtype=np.float64)
    _check(lib().orc_decode_matrix(_p(mat, _u8p), rows, cols, _p(w, _f64p)), "decode_matrix")
    return w


def rmsnorm(x, eps=RMS_EPS):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    _check(lib().orc_rmsnorm(_p(x, _f64p), x.size, eps, _p(out, _f64p)), "rmsnorm")
    return out


def silu(z):
    return lib().orc_silu(float(z))


def router_logits(xhat, R, bias=None):
    xhat = np.ascontiguousarray(xhat, dtype=np.float64)
    R = np.ascontiguousarray(R, dtype=np.uint16)
    E, H = R.shape
    out = np.empty(E, dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    _check(lib().orc_router_logits(_p(xhat, _f64p), _p(R, _u16p),
                                   None if b is None else _p(b, _f32p), E, H, _p(out, _f64p)),
           "router_logits")
    return out


def softmax_topk(logits, K, clamp=RENORM_CLAMP):
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    E = logits.size
    ids = np.empty(K, dtype=np.int32)
    w = np.empty(K, dtype=np.float64)
    p = np.empty(E, dtype=np.float64)
    _check(lib().orc_softmax_topk(_p(logits, _f64p), E, K, clamp, _p(ids, _i32p), _p(w, _f64p),
                                  _p(p, _f64p)), "softmax_topk")
    return ids, w, p


def expert(blob, xhat, H, FF):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    xhat = np.ascontiguousarray(xhat, dtype=np.float64)
    o = np.empty(H, dtype=np.float64)
    _check(lib().orc_expert(_p(blob, _u8p), _p(xhat, _f64p), H, FF, _p(o, _f64p)), "expert")
    return o


def route(x, R, K, bias=None, rmsnorm_flag=False, eps=RMS_EPS, clamp=RENORM_CLAMP):
    """Returns (ids [T][K] int32, w [T][K] f64, xhat [T][H] f64)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H = x.shape
    R = np.ascontiguousarray(R, dtype=np.uint16)
    E = R.shape[0]
    ids = np.empty((T, K), dtype=np.int32)
    w = np.empty((T, K), dtype=np.float64)
    xhat = np.empty((T, H), dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    _check(lib().orc_route(T, E, H, K, _p(x, _f32p), int(bool(rmsnorm_flag)), eps, _p(R, _u16p),
                           None if b is None else _p(b, _f32p), clamp, _p(ids, _i32p),
                           _p(w, _f64p), _p(xhat, _f64p)), "route")
    return ids, w, xhat


def experts(xhat, ids, blobs, E, H, FF):
    """blobs: mapping expert id -> uint8 array of blob bytes (only routed ones needed).
    Returns o [T*K][H] f64 in flat slot order t*K+k."""
    xhat = np.ascontiguousarray(xhat, dtype=np.float64)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    keep = {}
    ptrs = (ctypes.c_void_p * E)()
    for e in range(E):
        b = blobs.get(e) if hasattr(blobs, "get") else None
        if b is not None:
            arr = np.ascontiguousarray(b, dtype=np.uint8)
            keep[e] = arr
            ptrs[e] = arr.ctypes.data
    o = np.empty((T * K, H), dtype=np.float64)
    _check(lib().orc_experts(T, E, H, FF, K, _p(xhat, _f64p), _p(ids, _i32p), ptrs, _p(o, _f64p)),
           "experts")
    return o


def combine(o, w):
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, K = w.shape
    o = np.ascontiguousarray(o, dtype=np.float64)
    H = o.shape[-1]
    y = np.empty((T, H), dtype=np.float64)
    _check(lib().orc_combine(T, H, K, _p(o, _f64p), _p(w, _f64p), _p(y, _f64p)), "combine")
    return y


def layer(x, R, blobs, K, E, H, FF, bias=None, rmsnorm_flag=False):
    """Whole layer: returns (ids, w, y, xhat).  y excludes the residual."""
    ids, w, xhat = route(x, R, K, bias=bias, rmsnorm_flag=rmsnorm_flag)
    o = experts(xhat, ids, blobs, E, H, FF)
    y = combine(o, w)
    return ids, w, y, xhat


def num_threads():
    return int(lib().orc_num_threads())
