"""Correlated verify windows on the GPU (the first NEXT item): every token of
a T = 2, 3, 4 window gets, from the window call, bitwise the ids, weights and
layer output of its own T = 1 call -- the verifier contract of "Strata in the
source..." ("Drafting and verifying": a multi-token pass must give each token
what single-token decode gives it, bit for bit) -- and the window matches the
oracle to the parity bar.  Windows are drawn with inputs.draw_window and
screened for router near-ties.
"""
import numpy as np
import pytest

import harness as hz
import inputs
import oracle.screen as scr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hz.qm().lib()
    yield
    hz.drop_stores()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [2, 3, 4])
def test_correlated_window_equals_single_token_calls(T):
    seed = 800 + T
    print(f"case: correlated windows T={T}, seed {seed}", flush=True)
    st = inputs.Streams(seed)
    R = inputs.draw_router(st.router)
    wins, _ = scr.screened_windows(st, T, 6, R)
    store = hz.store(seed)
    distinct = []
    for i, x in enumerate(wins):
        ids, w, y, _ = hz.gpu_layer(x, R, store)
        distinct.append(np.unique(ids).size)
        for t in range(T):
            i1, w1, y1, _ = hz.gpu_layer(x[t:t + 1], R, store)
            assert np.array_equal(i1[0], ids[t]), (i, t)
            assert np.array_equal(w1[0], w[t]), (i, t)
            assert np.array_equal(y1[0], y[t]), (i, t)
        if i < 2:
            oids, ow, oy = hz.oracle_rows(x, R, seed, np.arange(T))
            hz.check(f"window T={T} #{i}", ids, w, y, oids, ow, oy)
    # correlated: fewer distinct experts than T independent tokens would give
    assert np.mean(distinct) < 10 * T - 2
