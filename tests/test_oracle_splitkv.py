"""Pins of the oracle's split-KV forward (few queries, many keys).

* The key ranges follow their definition: multiples of 128 keys, the last
  one shorter, covering every key exactly once, none empty, at most the
  requested number.
* One range is the plain quantized forward (the merge of a single part
  returns it unchanged).
* With several ranges the result stays within the method's accuracy of exact
  fp64 attention (cosine >= 0.999, as for the plain forward), and its
  log-sum-exp within the FP8 rounding of P of the exact one.
"""
import numpy as np
import pytest

import oracle
import workloads


@pytest.mark.parametrize("nk,n", [(1, 1), (127, 4), (128, 2), (4133, 5), (1000, 7), (32768, 64), (300, 64)])
def test_ranges(nk, n):
    rs = oracle.splitkv_ranges(nk, n)
    assert rs[0][0] == 0 and rs[-1][1] == nk
    assert all(a < b for a, b in rs)
    assert all(b == c for (_, b), (c, _) in zip(rs[:-1], rs[1:]))
    assert all(a % 128 == 0 for a, _ in rs)
    assert len(set(b - a for a, b in rs[:-1])) <= 1
    assert 1 <= len(rs) <= n


def _inputs(**kw):
    w = workloads.WORKLOADS["b2h8n4096d128"]
    inp = workloads.make_inputs(w, kw)
    return [inp[x].float().numpy() for x in ("q", "k", "v")]


@pytest.mark.parametrize("v_dtype", ["fp8", "fp16"])
def test_one_range_is_the_forward(v_dtype):
    q, k, v = _inputs(B=1, Hq=2, Hkv=1, Nq=9, Nk=700, d=96)
    s = oracle.reference_forward_splitkv(q, k, v, dtype="fp16", n_splits=1, gran="per_warp", v_dtype=v_dtype)
    r = oracle.reference_forward(q, k, v, dtype="fp16", gran="per_warp", v_dtype=v_dtype)
    np.testing.assert_array_equal(s["out"][0], r["out"][0])
    np.testing.assert_array_equal(s["lse"][0], r["lse"][0])


@pytest.mark.parametrize("n_splits", [2, 5])
def test_ranges_merge_to_attention(n_splits):
    q, k, v = _inputs(B=1, Hq=2, Hkv=2, Nq=12, Nk=1500, d=128)
    s = oracle.reference_forward_splitkv(q, k, v, dtype="fp16", n_splits=n_splits, gran="per_thread")
    ex = oracle.exact_forward(q, k, v)
    a, b = s["out"][0].ravel(), ex["out"][0].ravel()
    assert a @ b / np.linalg.norm(a) / np.linalg.norm(b) >= 0.999
    assert np.abs(s["lse"][0] - ex["lse"][0]).max() < 0.02
