"""An independent pure-Python/numpy fp64 implementation of the layer for tiny
shapes, used only to pin the oracle.  It shares nothing with oracle/: scales are
decoded by numpy's float16, router weights by numpy's float32 view, codes by a
bit-by-bit reading of the block, and the top-k by enumerating every ordering.
"""
import itertools
import math

import numpy as np

QK, BB = 64, 18


def block_weights(block):
    """The 64 weights of one 18-byte block: (code - 1) * scale."""
    d = float(np.frombuffer(bytes(block[0:2]), dtype="<f2")[0])
    bits = int.from_bytes(bytes(block[2:18]), "little")  # 128-bit code field
    return [(((bits >> (2 * i)) & 3) - 1) * d for i in range(QK)]


def matrix(mat_bytes, rows, cols):
    nb = cols // QK
    W = np.zeros((rows, cols))
    for r in range(rows):
        for b in range(nb):
            off = (r * nb + b) * BB
            W[r, b * QK:(b + 1) * QK] = block_weights(mat_bytes[off:off + BB])
    return W


def expert(blob, x, H, FF):
    m = H * FF // QK * BB
    Wg = matrix(blob[0:m], FF, H)
    Wu = matrix(blob[m:2 * m], FF, H)
    Wd = matrix(blob[2 * m:3 * m], H, FF)
    g = [sum(Wg[j, k] * x[k] for k in range(H)) for j in range(FF)]
    u = [sum(Wu[j, k] * x[k] for k in range(H)) for j in range(FF)]
    h = [g[j] / (1.0 + math.exp(-g[j])) * u[j] for j in range(FF)]
    return np.array([sum(Wd[r, j] * h[j] for j in range(FF)) for r in range(H)])


def bf16_values(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def stable_desc_order(keys):
    """First ordering, in lexicographic order of id tuples, whose keys never
    increase: ties therefore keep ascending id (a stable descending sort)."""
    E = len(keys)
    for perm in itertools.permutations(range(E)):
        if all(keys[perm[i]] >= keys[perm[i + 1]] for i in range(E - 1)):
            return list(perm)
    raise AssertionError("unreachable")


def layer(x, R_bits, blobs, K, H, FF, bias=None, rmsnorm=False, eps=1e-6, clamp=2.0 ** -14):
    """x [T][H] float32, R_bits [E][H] uint16 bf16 patterns, blobs list of bytes."""
    Rv = bf16_values(R_bits)
    E = Rv.shape[0]
    T = x.shape[0]
    ids = np.zeros((T, K), dtype=np.int32)
    w = np.zeros((T, K))
    y = np.zeros((T, H))
    for t in range(T):
        xv = [float(v) for v in x[t]]
        if rmsnorm:
            ms = sum(v * v for v in xv) / H
            xv = [v / math.sqrt(ms + eps) for v in xv]
        logits = [sum(Rv[e, k] * xv[k] for k in range(H)) + (0.0 if bias is None else float(bias[e]))
                  for e in range(E)]
        m = max(logits)
        ex = [math.exp(v - m) for v in logits]
        s = sum(ex)
        p = [v / s for v in ex]
        order = stable_desc_order([float(np.float32(v)) for v in p])
        sel = order[:K]
        den = max(sum(p[e] for e in sel), clamp)
        ids[t] = sel
        w[t] = [p[e] / den for e in sel]
        for k, e in enumerate(sel):
            y[t] += w[t, k] * expert(blobs[e], xv, H, FF)
    return ids, w, y
