"""Blob-store integrity on the GPU: the device checksums of a generated store
equal the checksums of the host generator's bytes, verification passes on the
store and names the first damaged blob of a copy with a flipped byte and with
two words that trade places."""
import numpy as np
import pytest

import harness as hz
import inputs
from test_store_check import checksum_np

pytestmark = pytest.mark.gpu

SEED, N = 7, 64


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m = hz.qm()
    m.lib()
    yield m
    hz.drop_stores()
    torch.cuda.empty_cache()


def test_checksums_and_verification(env):
    import torch
    m = env
    print(f"case: store seed {SEED}, first {N} blobs", flush=True)
    store = hz.store(SEED)
    expected = np.array([checksum_np(inputs.gen_blob(SEED, b)) for b in range(N)], dtype=np.uint64)
    sums = torch.empty(N, dtype=torch.int64, device="cuda")
    m.strata_moe_blob_checksums(store, N, sums)
    torch.cuda.synchronize()
    got = sums.cpu().numpy().view(np.uint64)
    assert np.array_equal(got, expected)
    assert m.strata_moe_verify_blobs(store, N, expected, sums) == -1

    bad = store[: N * m.BLOB].clone()
    bad[37 * m.BLOB + 12345] ^= 1                     # one bit of one byte in blob 37
    assert m.strata_moe_verify_blobs(bad, N, expected, sums) == 37
    words = bad[5 * m.BLOB: 6 * m.BLOB].view(torch.int64)
    a, b = words[10].clone(), words[20000].clone()
    assert not torch.equal(a, b)
    words[10], words[20000] = b, a                   # two words of blob 5 trade places
    assert m.strata_moe_verify_blobs(bad, N, expected, sums) == 5
    del bad, words
