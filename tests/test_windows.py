"""Correlated verify windows (the first NEXT item): the input recipe against
the pages' window figures, on the CPU with the oracle's routing.

"Strata in the source..." ("The plan: three destinations per expert") quotes
the distinct experts of a verify window as 1.75, 2.4 and 3.05 times one
token's for T = 2, 3, 4.  inputs.draw_window draws windows whose tokens share
a common component; this test checks that, routed by the oracle, they
reproduce those multiples (mean over 200 windows, within 4%).  A window
recipe with the wrong correlation (or uncorrelated tokens: 2.0 / 3.0 / 4.0)
fails it.
"""
import numpy as np
import pytest

import inputs
import oracle


@pytest.mark.parametrize("T,multiple", [(2, 1.75), (3, 2.4), (4, 3.05)])
def test_window_recipe_matches_the_pages_multiples(T, multiple):
    st = inputs.Streams(700 + T)
    R = inputs.draw_router(st.router)
    n = 200
    X = np.concatenate([inputs.draw_window(st.x, T) for _ in range(n)])
    ids, _, _ = oracle.route(X, R, inputs.K)
    distinct = [np.unique(ids[i * T:(i + 1) * T]).size for i in range(n)]
    got = float(np.mean(distinct)) / inputs.K
    assert abs(got - multiple) <= 0.04 * multiple, (T, got, multiple)


def test_window_tokens_are_standard_normal():
    st = inputs.Streams(9)
    w = np.concatenate([inputs.draw_window(st.x, 4) for _ in range(64)])
    assert w.dtype == np.float32 and w.shape == (256, inputs.H)
    assert abs(float(w.mean())) < 0.01 and abs(float(w.std()) - 1.0) < 0.01
