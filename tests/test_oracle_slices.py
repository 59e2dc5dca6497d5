"""Pins of the row-slice formulation used by the largest-chunk GPU tests -- CPU only.

tests/_slices.py computes the outputs of chunk rows [a, a + n) from a smaller oracle
call (cache extended by chunk keys 0..a-1). Checked against the full oracle call on
small random cases for every slice position; a planted off-by-one (cache extended by
keys 0..a) must fail.
"""
import numpy as np
import pytest

import oracle
from _slices import chunk_slice


def _case(G=2, P=5, C=9, D=8, seed=0):
    rng = np.random.default_rng(seed)
    n = lambda *s: rng.standard_normal(s)
    return dict(q=n(G, C, D), kc=n(C, D), vc=n(C, D), kp=n(P, D), vp=n(P, D), do=n(G, C, D),
                scale=1.0 / np.sqrt(D))


def _full(c):
    o, lse = oracle.group_fwd(c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    dq, dk, dv, _ = oracle.group_bwd(c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"],
                                     c["do"])
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("P", [0, 5])
def test_slices_equal_full_oracle(P):
    c = _case(P=P)
    o, lse, dq, dk, dv = _full(c)
    C = c["q"].shape[1]
    for a in range(C):
        for n in range(1, C - a + 1):
            so, sl, sdq, sdk, sdv = chunk_slice(c["q"], c["kc"], c["vc"], c["kp"], c["vp"],
                                                c["do"], c["scale"], a, n)
            np.testing.assert_allclose(so, o[:, a:a + n], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(sl, lse[:, a:a + n], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(sdq, dq[:, a:a + n], rtol=1e-12, atol=1e-13)
            if a + n == C:   # the tail keys see every row that reaches them
                np.testing.assert_allclose(sdk, dk[a:], rtol=1e-12, atol=1e-13)
                np.testing.assert_allclose(sdv, dv[a:], rtol=1e-12, atol=1e-13)


def test_planted_off_by_one_fails():
    c = _case(P=3, C=6)
    o = _full(c)[0]
    a, n = 2, 3
    kp2 = np.concatenate([c["kp"], c["kc"][:a + 1]])   # one chunk key too many
    vp2 = np.concatenate([c["vp"], c["vc"][:a + 1]])
    bad, _ = oracle.group_fwd(c["q"][:, a:a + n], c["kc"][a:a + n], c["vc"][a:a + n], kp2, vp2,
                              c["scale"])
    assert not np.allclose(bad, o[:, a:a + n], rtol=1e-6, atol=1e-8)
