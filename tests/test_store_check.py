"""The blob-store checksum (include/strata_moe.h, blob-store integrity) on the
CPU: the library's host function against the definition written out in numpy,
its sensitivity to a flipped byte and to two words trading places, and the
argument checks of the device entry points (each call fails validation on the
host, so nothing reaches a GPU)."""
import ctypes

import numpy as np
import pytest

GOLD = np.uint64(0x9E3779B97F4A7C15)


def checksum_np(blob):
    """sum_j mix(w_j + (j + 1) * GOLD) mod 2^64 over the little-endian 64-bit
    words w_j of the blob; mix is SplitMix64's output function."""
    w = np.ascontiguousarray(blob, dtype=np.uint8).view("<u8").astype(np.uint64)
    j = np.arange(w.size, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = w + (j + np.uint64(1)) * GOLD
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
        return int(np.sum(z, dtype=np.uint64))


@pytest.fixture(scope="module")
def m():
    import os
    import quantized_routed_expert_router_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    m.lib()
    return m


def test_mix_matches_the_published_splitmix64_outputs():
    """SplitMix64 seeded with 1234567: its state advances by GOLD and each
    output is mix(state); the first outputs of that generator as published
    with its reference implementation."""
    state = np.uint64(1234567)
    outs = []
    with np.errstate(over="ignore"):
        for _ in range(3):
            state = state + GOLD
            z = state
            z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
            z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
            outs.append(int(z ^ (z >> np.uint64(31))))
    assert outs == [6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_host_checksum_matches_the_definition(m):
    rng = np.random.default_rng(7)
    for _ in range(3):
        b = rng.integers(0, 256, m.BLOB, dtype=np.uint8)
        assert m.strata_moe_blob_checksum_host(b) == checksum_np(b)
    z = np.zeros(m.BLOB, np.uint8)
    assert m.strata_moe_blob_checksum_host(z) == checksum_np(z)


def test_checksum_sees_a_flipped_byte_and_a_swap(m):
    rng = np.random.default_rng(8)
    b = rng.integers(0, 256, m.BLOB, dtype=np.uint8)
    s0 = m.strata_moe_blob_checksum_host(b)
    for pos in (0, 1, 17, m.BLOB // 2, m.BLOB - 1):
        c = b.copy()
        c[pos] ^= 0x10
        assert m.strata_moe_blob_checksum_host(c) != s0, pos
    c = b.copy()
    w = c.view("<u8")
    w[[3, 1000]] = w[[1000, 3]]
    assert not np.array_equal(c, b)
    assert m.strata_moe_blob_checksum_host(c) != s0


def test_checksum_argument_checks(m):
    L = m.lib()
    fake = 0x100000   # never dereferenced: every call below fails validation first
    assert L.strata_moe_blob_checksums(None, 1, fake, None) == m.E_ARG
    assert L.strata_moe_blob_checksums(fake, 1, None, None) == m.E_ARG
    assert L.strata_moe_blob_checksums(fake, 0, fake, None) == m.E_SHAPE
    assert L.strata_moe_blob_checksums(fake, m.CHECK_BLOBS_MAX + 1, fake, None) == m.E_SHAPE
    assert L.strata_moe_blob_checksums(fake + 8, 1, fake, None) == m.E_ALIGN
    assert L.strata_moe_blob_checksums(fake, 1, fake + 4, None) == m.E_ALIGN
    first = ctypes.c_int64(5)
    ex = (ctypes.c_uint64 * 1)(0)
    assert L.strata_moe_verify_blobs(fake, 1, None, fake, ctypes.byref(first), None) == m.E_ARG
    assert L.strata_moe_verify_blobs(fake, 1, ex, fake, None, None) == m.E_ARG
    assert L.strata_moe_verify_blobs(fake, 0, ex, fake, ctypes.byref(first), None) == m.E_SHAPE
    assert first.value == -1
    assert L.strata_moe_blob_checksum_host(None) == 0
    assert "checksum" in m.strata_moe_status_string(m.E_CORRUPT)
