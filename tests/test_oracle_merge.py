"""Pins of the oracle's merge of partial attention results.

The merge (SageAttention deployment guide, pwwt.cn, sec. 4.1: return_lse
exists for Ring-Attention-style use) combines attention results over disjoint
key sets through their log-sum-exp values.  It is pinned to the mathematics:

* splitting the keys of a brute-force fp64 softmax attention (SciPy) into
  disjoint sets and merging the per-set results gives the attention over all
  keys, and their log-sum-exp, to rounding (any wrong weight, a missing
  normalisation or a sign error in the exponent breaks this);
* a single part is returned unchanged; equal log-sum-exps average the parts
  and add log S; a part with no keys (-inf) is ignored; a row with none gives
  0 and -inf; shifting every L_s by c shifts L by c and leaves out unchanged;
  the order of the parts does not matter.
"""
import numpy as np
import pytest
import scipy.special as sps

import oracle
import workloads


def _brute(q, k, v, sm):
    s = (q @ k.T) * sm
    return sps.softmax(s, axis=1) @ v, sps.logsumexp(s, axis=1)


@pytest.mark.parametrize("splits", [[0, 40, 100], [0, 1, 2, 77, 100], [0, 50, 51, 100]])
def test_merge_of_key_splits_equals_full_attention(splits):
    rng = np.random.default_rng(11)
    nq, nk, d = 37, 100, 24
    q, k, v = (rng.standard_normal(s) for s in ((nq, d), (nk, d), (nk, d)))
    sm = 1.0 / np.sqrt(d)
    full_o, full_l = _brute(q, k, v, sm)
    parts = [_brute(q, k[a:b], v[a:b], sm) for a, b in zip(splits[:-1], splits[1:])]
    o, L = oracle.merge_states(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(o, full_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, full_l, rtol=1e-14, atol=1e-12)


def test_single_part_is_identity():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((1, 9, 5))
    L = rng.standard_normal((1, 9))
    mo, ml = oracle.merge_states(o, L)
    np.testing.assert_array_equal(mo, o[0])
    np.testing.assert_allclose(ml, L[0], rtol=0, atol=1e-15)


def test_equal_lse_averages_parts():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((4, 6, 3))
    L = np.full((4, 6), 2.5)
    mo, ml = oracle.merge_states(o, L)
    np.testing.assert_allclose(mo, o.mean(axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(ml, 2.5 + np.log(4.0), rtol=0, atol=1e-15)


def test_empty_parts_and_rows():
    o = np.array([[[1.0, 2.0], [3.0, 4.0]], [[5.0, 6.0], [0.0, 0.0]]])
    L = np.array([[0.0, -np.inf], [-np.inf, -np.inf]])
    mo, ml = oracle.merge_states(o, L)
    np.testing.assert_array_equal(mo[0], [1.0, 2.0])        # part 1 of row 0 saw no key
    assert ml[0] == 0.0
    np.testing.assert_array_equal(mo[1], [0.0, 0.0])        # row 1 saw no key at all
    assert ml[1] == -np.inf


def test_shift_and_order_invariance():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((3, 8, 4))
    L = 5 * rng.standard_normal((3, 8))
    mo, ml = oracle.merge_states(o, L)
    so, sl = oracle.merge_states(o, L + 7.0)
    np.testing.assert_allclose(so, mo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sl, ml + 7.0, rtol=0, atol=1e-13)
    perm = [2, 0, 1]
    po, pl = oracle.merge_states(o[perm], L[perm])
    np.testing.assert_allclose(po, mo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(pl, ml, rtol=0, atol=1e-13)


def test_merge_input_generator_recipe():
    inp = workloads.make_merge_inputs(5, S=3, B=2, H=3, N=50, d=16, layout="NHD", empty_part_frac=0.2,
                                      empty_row_frac=0.1)
    o = inp["out_parts"].float().numpy()
    L = inp["lse_parts"].numpy()
    assert o.shape == (3, 2, 50, 3, 16) and L.shape == (3, 2, 3, 50)
    empty = np.isneginf(L)
    assert 0 < empty.mean() < 0.5
    assert np.all(o.transpose(0, 1, 3, 2, 4)[empty] == 0.0)
    assert np.isneginf(L).all(axis=0).any()                  # some rows have no key at all
