"""Pins for the CPU oracle against what the pages and the mathematics fix.

Every check compares the oracle with something other than itself: a value the
pages print (tests/golden/q2_0_format.json), a library decoder, a scalar
emulation of the quoted AVX-512 unpack, a closed form, or the independent
brute force in tests/bruteforce.py.
"""
import json
import math
import os

import numpy as np
import pytest

import bruteforce
import inputs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "q2_0_format.json")))


def g(name):
    return GOLD[name]["value"]


# ---------------------------------------------------------------- byte budget
def test_blob_and_store_sizes(orc):
    H, FF = g("H"), g("FF")
    blob = orc.blob_bytes(H, FF)
    assert blob == g("blob_bytes") == 1382400
    assert blob * 8 / (3 * H * FF) == g("bits_per_weight")
    assert blob * g("layers") * g("experts_per_layer") == g("store_bytes")
    per_token = g("layers") * g("top_k") * blob
    assert g("layers") * g("top_k") == g("blobs_per_token")
    assert round(per_token / 1e6, 1) == g("expert_bytes_per_token_MB")
    assert round(g("experts_per_layer") * blob / 1e6) == g("one_layer_store_MB")
    assert orc.blob_bytes(64, 128) == 6912  # the tiny brute-force instance
    assert orc.blob_bytes(2560, 600) == 0  # FF not a multiple of QK is refused


# ---------------------------------------------------------------- decoders
def test_half_decoder_all_patterns(orc):
    pats = np.arange(65536, dtype=np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decoder_all_patterns(orc):
    pats = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):   # signalling-NaN patterns widen to NaN
        ref = (pats << 16).view(np.float32).astype(np.float64)
    got = np.array([orc.bf16_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def multishift_unpack(code_bytes):
    """Scalar emulation of the quoted unpack: load 16 bytes as 8 u16, widen
    each to a qword, multishift with the control from the page (each output
    byte j of a qword takes the 8 bits starting at bit ctrl_j, wrapping), then
    AND with 3.  Returns the 64 lanes in vector order."""
    ctrl = int(g("multishift_control"), 16)
    u16 = [int.from_bytes(code_bytes[2 * q:2 * q + 2], "little") for q in range(8)]
    out = []
    for q in range(8):
        qw = u16[q]  # zero-extended to 64 bits
        for j in range(8):
            c = (ctrl >> (8 * j)) & 0x3F
            rot = ((qw >> c) | (qw << (64 - c))) & ((1 << 64) - 1) if c else qw
            out.append((rot & 0xFF) & 3)
    return out


def test_code_bit_order_matches_quoted_unpack(orc):
    rng = np.random.default_rng(11)
    for _ in range(200):
        blk = bytes([0, 0x3C]) + bytes(rng.integers(0, 256, 16, dtype=np.uint8))
        assert orc.q2_codes(blk) == multishift_unpack(blk[2:])


def test_hand_built_blocks(orc):
    one = bytes([0x00, 0x3C])  # fp16 1.0, little-endian
    vals = g("code_values")
    # all codes 3 -> 2 * d
    w = orc.decode_matrix(one + bytes([0xFF] * 16), 1, 64)
    assert np.all(w == 2.0 * vals["3"] / 2)
    # repeating codes 0,1,2,3 (byte 0b11100100) -> -1, 0, 1, 2
    w = orc.decode_matrix(one + bytes([0xE4] * 16), 1, 64)[0]
    assert list(w[:4]) == [vals["0"], vals["1"], vals["2"], vals["3"]]
    assert np.array_equal(w, np.tile([-1.0, 0.0, 1.0, 2.0], 16))
    # all codes 1 -> exact zero
    assert np.all(orc.decode_matrix(bytes([0x00, 0x38]) + bytes([0x55] * 16), 1, 64) == 0.0)
    # the scale sits in bytes 0-1: 0x3800 = 0.5, codes 2 -> +0.5
    w = orc.decode_matrix(bytes([0x00, 0x38]) + bytes([0xAA] * 16), 1, 64)
    assert np.all(w == 0.5)
    # the last code byte holds codes 60..63; first code byte codes 0..3
    blk = bytearray(one + bytes([0x55] * 16))
    blk[17] = 0xFF
    w = orc.decode_matrix(bytes(blk), 1, 64)[0]
    assert np.all(w[:60] == 0.0) and np.all(w[60:] == 2.0)
    blk = bytearray(one + bytes([0x55] * 16))
    blk[2] = 0x54  # code 0 -> 0
    w = orc.decode_matrix(bytes(blk), 1, 64)[0]
    assert w[0] == -1.0 and np.all(w[1:] == 0.0)


def test_matrix_rows_are_blocked_along_input(orc):
    rows, cols = 3, 128
    mat = bytearray()
    for r in range(rows):
        for b in range(2):
            d = np.float16(0.25 * (r + 1) * (b + 1)).view(np.uint16)
            mat += int(d).to_bytes(2, "little") + bytes([0xAA] * 16)
    w = orc.decode_matrix(bytes(mat), rows, cols)
    for r in range(rows):
        assert np.all(w[r, :64] == 0.25 * (r + 1))
        assert np.all(w[r, 64:] == 0.5 * (r + 1))


# ---------------------------------------------------------------- router
def test_router_one_hot_gives_a_column(orc):
    rng = np.random.default_rng(3)
    R = inputs.draw_router(rng, e=16, h=128)
    Rv = (R.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for j in (0, 5, 127):
        x = np.zeros(128)
        x[j] = 1.0
        assert np.array_equal(orc.router_logits(x, R), Rv[:, j])
    bias = rng.standard_normal(16).astype(np.float32)
    x = np.zeros(128)
    x[7] = 1.0
    assert np.array_equal(orc.router_logits(x, R, bias), Rv[:, 7] + bias.astype(np.float64))


def test_softmax_topk_invariants(orc):
    from scipy.special import softmax
    rng = np.random.default_rng(5)
    for _ in range(50):
        lg = rng.standard_normal(512) * 1.5
        ids, w, p = orc.softmax_topk(lg, 10)
        assert np.allclose(p, softmax(lg), rtol=1e-14, atol=0)
        assert len(set(ids.tolist())) == 10
        assert abs(w.sum() - 1.0) < 1e-14
        assert np.all(np.diff(w) <= 0)
        # the selected ids are exactly the 10 largest logits, in descending order
        assert list(ids) == list(np.argsort(-lg, kind="stable")[:10])
        # renormalised weights equal the softmax over the 10 selected logits
        assert np.allclose(w, softmax(lg[ids]), rtol=1e-13, atol=0)
    lg = rng.standard_normal(64)
    ids, w, p = orc.softmax_topk(lg, 64)  # k = E: the dense softmax mixture
    assert np.allclose(w[np.argsort(ids)], softmax(lg), rtol=1e-13)
    ids, w, _ = orc.softmax_topk(lg, 1)  # k = 1: weight 1
    assert w[0] == 1.0 and ids[0] == int(np.argmax(lg))


def test_stable_ties(orc):
    lg = np.linspace(2.0, -2.0, 512)
    lg[[3, 7, 9, 11]] = lg[2]  # a four-way tie inside the top-10
    ids, _, _ = orc.softmax_topk(lg, 10)
    assert list(ids[:5]) == [0, 1, 2, 3, 7]
    # a tie straddling ranks 10 and 11: the lower id is kept
    lg = -np.arange(512, dtype=np.float64)
    lg[400] = lg[9]
    ids, _, _ = orc.softmax_topk(lg, 10)
    assert list(ids) == list(range(10))
    lg[5] = lg[9]  # now 5, 9 and 400 tie; 5 moves to the tie group's first slot
    ids, _, _ = orc.softmax_topk(lg, 10)
    assert list(ids) == [0, 1, 2, 3, 4, 6, 7, 8, 5, 9]
    # duplicated router rows through the GEMV tie exactly and keep id order
    rng = np.random.default_rng(8)
    R = inputs.draw_router(rng, e=32, h=256)
    R[20] = R[4]
    R[31] = R[4]
    x = rng.standard_normal(256)
    lgr = orc.router_logits(x, R)
    assert lgr[4] == lgr[20] == lgr[31]
    ids, _, _ = orc.softmax_topk(lgr, 32)
    pos = [list(ids).index(e) for e in (4, 20, 31)]
    assert pos == sorted(pos) and pos[2] - pos[0] == 2


def test_renorm_clamp_reading(orc):
    # With a uniform softmax over 32768 experts each p = 2^-15 < 2^-14, so
    # for k = 1 the clamp is active and the weight is p / clamp = 0.5.
    ids, w, _ = orc.softmax_topk(np.zeros(32768), 1, clamp=2.0 ** -14)
    assert ids[0] == 0 and w[0] == 0.5
    # For the workload's E = 512, k = 10 it is provably inactive: the top-10
    # mass is at least 10/512.
    ids, w, p = orc.softmax_topk(np.zeros(512), 10)
    assert abs(w.sum() - 1.0) < 1e-15


# ---------------------------------------------------------------- norm and expert
def test_rmsnorm_closed_forms(orc):
    for c in (0.5, 3.0, -2.0):
        x = np.full(2560, c)
        assert np.allclose(orc.rmsnorm(x), c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    x = np.array([3.0, 4.0])
    assert np.allclose(orc.rmsnorm(x), x / math.sqrt(12.5 + 1e-6), rtol=1e-15)


def _uniform_matrix(rows, cols, code_byte, scale):
    d = int(np.float16(scale).view(np.uint16)).to_bytes(2, "little")
    return (d + bytes([code_byte] * 16)) * (rows * cols // 64)


def test_expert_closed_form(orc):
    H, FF = 128, 64
    # gate weights all +1, up all +0.5, down all 2 * 0.25 = 0.5
    blob = (_uniform_matrix(FF, H, 0xAA, 1.0) + _uniform_matrix(FF, H, 0xAA, 0.5)
            + _uniform_matrix(H, FF, 0xFF, 0.25))
    rng = np.random.default_rng(2)
    x = rng.standard_normal(H) * 0.1
    S = x.sum()
    h = S / (1 + math.exp(-S)) * 0.5 * S
    o = orc.expert(np.frombuffer(blob, np.uint8), x, H, FF)
    assert np.allclose(o, 0.5 * FF * h, rtol=1e-13)
    # zero-valued experts (all codes 1) give exactly zero
    zero = (_uniform_matrix(FF, H, 0x55, 0.03) * 2 + _uniform_matrix(H, FF, 0x55, 0.03))
    assert np.all(orc.expert(np.frombuffer(zero, np.uint8), x, H, FF) == 0.0)


def test_one_hot_gate_up_columns(orc):
    """With down = identity-like rows, o picks single h entries; with one-hot x,
    g and u are columns of the dequantised gate and up matrices."""
    H, FF = 64, 64
    rng = np.random.default_rng(4)
    gate = inputs.gen_blob(9, 0, h=H, ff=FF)[: H * FF // 64 * 18]
    up = inputs.gen_blob(9, 1, h=H, ff=FF)[: H * FF // 64 * 18]
    # down row r has weight 1 at column r only is not expressible in Q2_0 with
    # one scale per 64, so use all-ones down: o_r = sum_j h_j for every r
    down = np.frombuffer(_uniform_matrix(H, FF, 0xAA, 1.0), np.uint8)
    blob = np.concatenate([gate, up, down])
    Wg = bruteforce.matrix(bytes(gate), FF, H)
    Wu = bruteforce.matrix(bytes(up), FF, H)
    for j in (0, 17, 63):
        x = np.zeros(H)
        x[j] = 1.0
        gcol, ucol = Wg[:, j], Wu[:, j]
        hsum = sum(gv / (1 + math.exp(-gv)) * uv for gv, uv in zip(gcol, ucol))
        o = orc.expert(blob, x, H, FF)
        assert np.allclose(o, hsum, rtol=1e-12, atol=1e-15)
    del rng


# ---------------------------------------------------------------- whole layer
@pytest.mark.parametrize("K", [1, 2, 8])
def test_bruteforce_tiny_instance(orc, K):
    E, H, FF, T = 8, 64, 128, 3
    seed = 100 + K
    st = inputs.Streams(seed)
    x = inputs.draw_x(st.x, T, h=H)
    R = inputs.draw_router(st.router, e=E, h=H)
    blobs = {e: inputs.gen_blob(seed, e, h=H, ff=FF) for e in range(E)}
    ids, w, y, _ = orc.layer(x, R, blobs, K, E, H, FF)
    bids, bw, by = bruteforce.layer(x, R, [bytes(blobs[e]) for e in range(E)], K, H, FF)
    assert np.array_equal(ids, bids)
    assert np.allclose(w, bw, rtol=1e-13, atol=0)
    assert np.allclose(y, by, rtol=1e-11, atol=1e-14 * np.abs(by).max())


def test_bruteforce_tiny_with_ties_bias_and_norm(orc):
    E, H, FF, T, K = 8, 64, 128, 3, 4
    st = inputs.Streams(77)
    x = inputs.draw_x(st.x, T, h=H) * 3.0
    R = inputs.draw_router(st.router, e=E, h=H)
    R[5] = R[1]  # duplicated rows tie exactly
    R[6] = R[1]
    bias = inputs.draw_zipf_bias(st.bias, e=E)
    bias[5] = bias[1]
    bias[6] = bias[1]
    blobs = {e: inputs.gen_blob(77, e, h=H, ff=FF) for e in range(E)}
    ids, w, y, _ = orc.layer(x, R, blobs, K, E, H, FF, bias=bias, rmsnorm_flag=True)
    bids, bw, by = bruteforce.layer(x, R, [bytes(blobs[e]) for e in range(E)], K, H, FF,
                                    bias=bias, rmsnorm=True)
    assert np.array_equal(ids, bids)
    assert np.allclose(w, bw, rtol=1e-13, atol=0)
    assert np.allclose(y, by, rtol=1e-11, atol=1e-14 * np.abs(by).max())


def test_identical_experts_give_one_output(orc):
    E, H, FF = 16, 64, 128
    st = inputs.Streams(21)
    x = inputs.draw_x(st.x, 2, h=H)
    R = inputs.draw_router(st.router, e=E, h=H)
    same = inputs.gen_blob(21, 0, h=H, ff=FF)
    blobs = {e: same for e in range(E)}
    ids, w, y, xhat = orc.layer(x, R, blobs, 10, E, H, FF)
    for t in range(2):
        o1 = orc.expert(same, xhat[t], H, FF)
        assert np.allclose(y[t], o1, rtol=1e-13, atol=1e-16)


def test_combine_is_weighted_sum_in_routing_order(orc):
    rng = np.random.default_rng(6)
    o = rng.standard_normal((3 * 10, 32))
    w = rng.random((3, 10))
    y = orc.combine(o, w)
    ref = np.einsum("tk,tkh->th", w, o.reshape(3, 10, 32))
    assert np.allclose(y, ref, rtol=1e-14)


def test_bruteforce_tall_down_matrix(orc):
    """H > FF, as in the workload (2560 > 640): down has more rows than its
    input width, so a transposed or wrapped down index shows here."""
    E, H, FF, T, K = 4, 128, 64, 2, 2
    st = inputs.Streams(55)
    x = inputs.draw_x(st.x, T, h=H)
    R = inputs.draw_router(st.router, e=E, h=H)
    blobs = {e: inputs.gen_blob(55, e, h=H, ff=FF) for e in range(E)}
    ids, w, y, _ = orc.layer(x, R, blobs, K, E, H, FF)
    bids, bw, by = bruteforce.layer(x, R, [bytes(blobs[e]) for e in range(E)], K, H, FF)
    assert np.array_equal(ids, bids)
    assert np.allclose(w, bw, rtol=1e-13, atol=0)
    assert np.allclose(y, by, rtol=1e-11, atol=1e-14 * np.abs(by).max())
