"""Routed-expert MoE layer on MI355X: Python binding of libstrata_moe.so.

Argument marshalling only -- every step of the layer runs in the HIP kernels
behind the C ABI of include/strata_moe.h.  Functions carry the C names and take
torch tensors on the GPU (their device pointers are passed through) plus an
optional hipStream_t handle (default: torch's current stream).  If the library
is not built, importing works but the first call raises: there is no CPU
fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstrata_moe.so")

H, FF, E, K, QK, BB = 2560, 640, 512, 10, 64, 18
BLOB = 1382400
T_MAX = 8192
LOOKAHEAD_T_MAX = 8
RMSNORM, RESIDUAL, INT8 = 1, 2, 4
OK, E_ARG, E_SHAPE, E_WORKSPACE, E_HIP, E_ALIGN, E_CORRUPT = 0, -1, -2, -3, -4, -5, -6
CHECK_BLOBS_MAX = 1 << 24

EXPORTS = ("strata_moe_blob_bytes", "strata_moe_workspace_bytes", "strata_moe_route",
           "strata_moe_group", "strata_moe_experts", "strata_moe_combine", "strata_moe_layer",
           "strata_moe_layer_lookahead", "strata_moe_time_next_kernel",
           "strata_moe_read_status", "strata_moe_clear_status", "strata_moe_set_wait_limit",
           "strata_moe_layer_static", "strata_moe_status_string", "strata_moe_blob_checksums",
           "strata_moe_blob_checksum_host", "strata_moe_verify_blobs")
STATIC_T_MAX = 64
STATUS_WAIT_TIMEOUT = 1

_lib = None


class StrataError(RuntimeError):
    def __init__(self, fn, rc):
        super().__init__(f"{fn} failed: {rc} ({strata_moe_status_string(rc)})")
        self.rc = rc


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the layer has no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.strata_moe_blob_bytes.restype = sz
        L.strata_moe_blob_bytes.argtypes = []
        L.strata_moe_workspace_bytes.restype = sz
        L.strata_moe_workspace_bytes.argtypes = [i32]
        L.strata_moe_route.restype = i32
        L.strata_moe_route.argtypes = [vp, i32, vp, vp, i32, vp, vp, vp, sz, vp]
        L.strata_moe_group.restype = i32
        L.strata_moe_group.argtypes = [vp, i32, vp, vp, vp, vp, sz, vp]
        L.strata_moe_experts.restype = i32
        L.strata_moe_experts.argtypes = [vp, i32, vp, vp, vp, vp, i32, vp, vp, sz, vp]
        L.strata_moe_combine.restype = i32
        L.strata_moe_combine.argtypes = [vp, vp, i32, i32, vp, vp]
        L.strata_moe_layer.restype = i32
        L.strata_moe_layer.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        L.strata_moe_layer_lookahead.restype = i32
        L.strata_moe_layer_lookahead.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                                 vp, vp, vp, sz, vp]
        L.strata_moe_time_next_kernel.restype = i32
        L.strata_moe_time_next_kernel.argtypes = [vp, vp]
        L.strata_moe_layer_static.restype = i32
        L.strata_moe_layer_static.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp]
        L.strata_moe_read_status.restype = i32
        L.strata_moe_read_status.argtypes = [vp, sz, ctypes.POINTER(ctypes.c_int32), vp]
        L.strata_moe_clear_status.restype = i32
        L.strata_moe_clear_status.argtypes = [vp, sz, vp]
        L.strata_moe_set_wait_limit.restype = i32
        L.strata_moe_set_wait_limit.argtypes = [i32]
        L.strata_moe_status_string.restype = ctypes.c_char_p
        L.strata_moe_status_string.argtypes = [i32]
        i64, u64p = ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64)
        L.strata_moe_blob_checksums.restype = i32
        L.strata_moe_blob_checksums.argtypes = [vp, i64, vp, vp]
        L.strata_moe_blob_checksum_host.restype = ctypes.c_uint64
        L.strata_moe_blob_checksum_host.argtypes = [vp]
        L.strata_moe_verify_blobs.restype = i32
        L.strata_moe_verify_blobs.argtypes = [vp, i64, u64p, vp, ctypes.POINTER(i64), vp]
        _lib = L
    return _lib


def _p(t, dtype=None):
    """Device pointer of a tensor (None passes NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _p_router(t):
    import torch
    if t is not None and t.dtype not in (torch.int16, torch.bfloat16):
        raise TypeError("router must hold bf16 bit patterns (int16 or bfloat16 tensor)")
    return _p(t)


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t):
    return t.numel() * t.element_size()


def _shape(name, t, shape):
    """Raise ValueError unless tensor t (or None, when allowed by the caller)
    has exactly `shape`: undersized buffers never reach the kernels."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _opt_shape(name, t, shape):
    if t is not None:
        _shape(name, t, shape)


def _min_numel(name, t, n):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dim() != 1 or t.numel() < n:
        raise ValueError(f"{name} must be 1-D with at least {n} elements, got {tuple(t.shape)}")


def _tokens(x):
    """T of an activation tensor x [T][H] (checked against the layer width)."""
    if x is None or x.dim() != 2 or x.shape[1] != H:
        raise ValueError(f"x must have shape (T, {H}), got "
                         f"{None if x is None else tuple(x.shape)}")
    T = int(x.shape[0])
    if not 1 <= T <= T_MAX:
        raise ValueError(f"T = {T} outside 1..{T_MAX}")
    return T


def _router_shape(name, R):
    if R is None or R.numel() != E * H or R.dim() not in (1, 2) or (
            R.dim() == 2 and tuple(R.shape) != (E, H)):
        raise ValueError(f"{name} must hold {E} x {H} bf16 values, got "
                         f"{None if R is None else tuple(R.shape)}")


def _store_shape(name, blobs):
    _min_numel(name, blobs, E * BLOB)


def _ws_shape(ws, T):
    need = strata_moe_workspace_bytes(T)
    if ws is None or ws.dim() != 1 or _nbytes(ws) < need:
        raise ValueError(f"workspace must be a 1-D tensor of at least {need} bytes for T = {T}")


def _check(fn, rc):
    if rc != OK:
        raise StrataError(fn, rc)


def strata_moe_status_string(rc):
    return lib().strata_moe_status_string(int(rc)).decode()


def strata_moe_blob_bytes():
    return int(lib().strata_moe_blob_bytes())


def strata_moe_workspace_bytes(T):
    return int(lib().strata_moe_workspace_bytes(int(T)))


def workspace(T, device="cuda"):
    """A workspace tensor sized for T tokens (torch allocations are 256-aligned),
    zero-filled so that its status word starts clear."""
    import torch
    n = strata_moe_workspace_bytes(T)
    if n == 0:
        raise StrataError("strata_moe_workspace_bytes", E_SHAPE)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def strata_moe_read_status(ws, stream=None):
    """Synchronise the stream and return the workspace's status word (bits
    STATUS_*; 0 when every call since the last clear completed normally)."""
    v = ctypes.c_int32(0)
    rc = lib().strata_moe_read_status(_p(ws), _nbytes(ws), ctypes.byref(v), _s(stream))
    _check("strata_moe_read_status", rc)
    return int(v.value)


def strata_moe_clear_status(ws, stream=None):
    _check("strata_moe_clear_status", lib().strata_moe_clear_status(_p(ws), _nbytes(ws), _s(stream)))


def strata_moe_set_wait_limit(polls):
    """Bound of the decode experts kernel's wait (0 restores the default)."""
    _check("strata_moe_set_wait_limit", lib().strata_moe_set_wait_limit(int(polls)))


def _blob_count(blobs, nblobs):
    """Check that the uint8 device tensor `blobs` holds nblobs blobs."""
    import torch
    if blobs is None or blobs.dtype != torch.uint8:
        raise TypeError("blobs must be a uint8 tensor")
    nblobs = int(nblobs)
    if nblobs < 1 or nblobs > CHECK_BLOBS_MAX:
        raise ValueError(f"nblobs must be in 1..{CHECK_BLOBS_MAX}, got {nblobs}")
    if blobs.numel() < nblobs * BLOB:
        raise ValueError(f"blobs holds {blobs.numel()} bytes, fewer than {nblobs} blobs")
    return nblobs


def strata_moe_blob_checksums(blobs, nblobs, sums, stream=None):
    """Enqueue the 64-bit checksum of each of the first nblobs blobs of the
    device store `blobs` into the int64 device tensor sums [nblobs] (bit
    patterns of the uint64 checksums)."""
    import torch
    n = _blob_count(blobs, nblobs)
    if sums.dtype != torch.int64:
        raise TypeError("sums must be an int64 tensor (uint64 bit patterns)")
    _min_numel("sums", sums, n)
    _check("strata_moe_blob_checksums",
           lib().strata_moe_blob_checksums(_p(blobs), n, _p(sums), _s(stream)))


def strata_moe_blob_checksum_host(blob):
    """Checksum of one blob in host memory (a numpy uint8 array of BLOB bytes)."""
    import numpy as np
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    if b.size != BLOB:
        raise ValueError(f"a blob is {BLOB} bytes, got {b.size}")
    return int(lib().strata_moe_blob_checksum_host(b.ctypes.data))


def strata_moe_verify_blobs(blobs, nblobs, expected, sums, stream=None):
    """Synchronously compare the first nblobs device blobs with `expected`
    (host numpy uint64 [nblobs]); sums is device scratch (int64 [nblobs]).
    Returns -1 if every checksum matches, else the first differing index
    (the C call returned STRATA_E_CORRUPT); raises on any other error."""
    import numpy as np
    import torch
    n = _blob_count(blobs, nblobs)
    ex = np.ascontiguousarray(expected, dtype=np.uint64)
    if ex.size < n:
        raise ValueError(f"expected holds {ex.size} checksums, fewer than {n}")
    if sums.dtype != torch.int64:
        raise TypeError("sums must be an int64 tensor (uint64 bit patterns)")
    _min_numel("sums", sums, n)
    first = ctypes.c_int64(-2)
    rc = lib().strata_moe_verify_blobs(_p(blobs), n, ex.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                       _p(sums), ctypes.byref(first), _s(stream))
    if rc == E_CORRUPT:
        return int(first.value)
    _check("strata_moe_verify_blobs", rc)
    return -1


def strata_moe_route(x, router, ids, w, ws, bias=None, flags=0, stream=None):
    import torch
    T = _tokens(x)
    _router_shape("router", router)
    _opt_shape("bias", bias, (E,))
    _shape("ids", ids, (T, K))
    _shape("w", w, (T, K))
    _ws_shape(ws, T)
    rc = lib().strata_moe_route(_p(x, torch.float32), T, _p_router(router),
                                _p(bias, torch.float32), flags, _p(ids, torch.int32),
                                _p(w, torch.float32), _p(ws), _nbytes(ws), _s(stream))
    _check("strata_moe_route", rc)


def strata_moe_group(ids, offsets, slots, active, ws, stream=None):
    import torch
    if ids is None or ids.dim() != 2 or ids.shape[1] != K or not 1 <= ids.shape[0] <= T_MAX:
        raise ValueError(f"ids must have shape (T, {K}) with 1 <= T <= {T_MAX}")
    T = int(ids.shape[0])
    _shape("offsets", offsets, (E + 1,))
    _shape("slots", slots, (T * K,))
    _shape("active", active, (E + 1,))
    _ws_shape(ws, T)
    rc = lib().strata_moe_group(_p(ids, torch.int32), T, _p(offsets, torch.int32),
                                _p(slots, torch.int32), _p(active, torch.int32), _p(ws),
                                _nbytes(ws), _s(stream))
    _check("strata_moe_group", rc)


def strata_moe_experts(x, blobs, offsets, slots, active, out, ws, flags=0, stream=None):
    import torch
    T = _tokens(x)
    _store_shape("blobs", blobs)
    _shape("offsets", offsets, (E + 1,))
    _shape("slots", slots, (T * K,))
    _shape("active", active, (E + 1,))
    _shape("out", out, (T * K, H))
    _ws_shape(ws, T)
    rc = lib().strata_moe_experts(_p(x, torch.float32), T, _p(blobs, torch.uint8),
                                  _p(offsets, torch.int32), _p(slots, torch.int32),
                                  _p(active, torch.int32), flags, _p(out, torch.float32), _p(ws),
                                  _nbytes(ws), _s(stream))
    _check("strata_moe_experts", rc)


def strata_moe_combine(out, w, y, flags=0, stream=None):
    import torch
    T = _tokens(y)
    _shape("out", out, (T * K, H))
    _shape("w", w, (T, K))
    rc = lib().strata_moe_combine(_p(out, torch.float32), _p(w, torch.float32), T, flags,
                                  _p(y, torch.float32), _s(stream))
    _check("strata_moe_combine", rc)


def strata_moe_time_next_kernel(start=None, stop=None):
    """Arm the next experts/layer call to record two torch.cuda.Event objects
    (enable_timing=True) around its dominant kernel; None, None disarms."""
    def handle(ev):
        if ev is None:
            return None
        if not ev.cuda_event:
            raise ValueError("record the event once before passing it (its HIP event is lazy)")
        return int(ev.cuda_event)
    rc = lib().strata_moe_time_next_kernel(handle(start), handle(stop))
    _check("strata_moe_time_next_kernel", rc)


def strata_moe_layer(x, router, blobs, ws, bias=None, flags=0, y=None, ids=None, w=None,
                     stream=None):
    import torch
    T = _tokens(x)
    _router_shape("router", router)
    _store_shape("blobs", blobs)
    _opt_shape("bias", bias, (E,))
    _opt_shape("y", y, (T, H))
    _opt_shape("ids", ids, (T, K))
    _opt_shape("w", w, (T, K))
    _ws_shape(ws, T)
    rc = lib().strata_moe_layer(_p(x, torch.float32), T, _p_router(router),
                                _p(bias, torch.float32), _p(blobs, torch.uint8), flags,
                                _p(y, torch.float32), _p(ids, torch.int32), _p(w, torch.float32),
                                _p(ws), _nbytes(ws), _s(stream))
    _check("strata_moe_layer", rc)


def strata_moe_layer_static(x, router, blobs, bias=None, flags=0, y=None, ids=None, w=None,
                            stream=None):
    """strata_moe_layer on the library's static per-GPU workspace (no
    workspace argument, nothing allocated; T <= STATIC_T_MAX; calls on one GPU
    must not overlap)."""
    import torch
    T = _tokens(x)
    if T > STATIC_T_MAX:
        raise ValueError(f"T = {T} exceeds the static workspace's {STATIC_T_MAX} tokens")
    _router_shape("router", router)
    _store_shape("blobs", blobs)
    _opt_shape("bias", bias, (E,))
    _opt_shape("y", y, (T, H))
    _opt_shape("ids", ids, (T, K))
    _opt_shape("w", w, (T, K))
    rc = lib().strata_moe_layer_static(_p(x, torch.float32), T, _p_router(router),
                                       _p(bias, torch.float32), _p(blobs, torch.uint8), flags,
                                       _p(y, torch.float32), _p(ids, torch.int32),
                                       _p(w, torch.float32), _s(stream))
    _check("strata_moe_layer_static", rc)


def strata_moe_layer_lookahead(x, router, blobs, ws, router_next, blobs_next, bias=None,
                               bias_next=None, flags=0, y=None, ids=None, w=None, pred=None,
                               hint=None, stream=None):
    import torch
    T = _tokens(x)
    _router_shape("router", router)
    _router_shape("router_next", router_next)
    _store_shape("blobs", blobs)
    _store_shape("blobs_next", blobs_next)
    _opt_shape("bias", bias, (E,))
    _opt_shape("bias_next", bias_next, (E,))
    _opt_shape("y", y, (T, H))
    _opt_shape("ids", ids, (T, K))
    _opt_shape("w", w, (T, K))
    _opt_shape("pred", pred, (T, K))
    _opt_shape("hint", hint, (T, K))
    _ws_shape(ws, T)
    rc = lib().strata_moe_layer_lookahead(
        _p(x, torch.float32), T, _p_router(router), _p(bias, torch.float32),
        _p(blobs, torch.uint8), flags, _p(y, torch.float32), _p(ids, torch.int32),
        _p(w, torch.float32), _p_router(router_next), _p(bias_next, torch.float32),
        _p(blobs_next, torch.uint8), _p(pred, torch.int32), _p(hint, torch.int32), _p(ws),
        _nbytes(ws), _s(stream))
    _check("strata_moe_layer_lookahead", rc)
