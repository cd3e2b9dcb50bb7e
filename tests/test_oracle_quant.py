"""Pins of the oracle's quantization steps (INT8 Q/K groups, FP8 V, exact means).

Sources: SageAttention deployment guide (pwwt.cn), sec. 1 (Q, K -> INT8 with
per-block / per-thread scales; V -> FP8) and sec. 4.2 (qk_quant_gran, smooth_k
subtracts K's mean along the sequence, smooth_v subtracts V's mean).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8_quantizer_cases.txt")


def _golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        vals, codes, scale = line.split("|")
        cases.append(([float(t) for t in vals.split(",")], [int(t) for t in codes.split(",")], float(scale)))
    return cases


@pytest.mark.parametrize("vals,codes,scale", _golden_cases())
def test_int8_hand_cases(vals, codes, scale):
    x = np.array(vals, dtype=np.float32)[:, None]          # one column, one group
    c, s = oracle.quant_int8(x, len(vals), len(vals))
    assert list(c[:, 0]) == codes
    assert s[0] == np.float32(scale)


def test_int8_matches_library_rounding():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((96, 64)).astype(np.float32) * rng.uniform(0.01, 50, size=(96, 1)).astype(np.float32)
    for g in (1, 16, 32, 64):
        c, s = oracle.quant_int8(x, 96, g)
        xt = torch.from_numpy(x)
        for gi in range(96 // g):
            blk = xt[gi * g:(gi + 1) * g]
            amax = blk.abs().max()
            inv = torch.tensor(127.0, dtype=torch.float32) / amax
            ref = torch.round(blk * inv).clamp(-127, 127).to(torch.int8).numpy()   # torch.round: half to even
            assert np.array_equal(c[gi * g:(gi + 1) * g], ref)
            assert s[gi] == (amax / torch.tensor(127.0)).item()


def test_int8_power_of_two_invariance_and_locality():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    c0, s0 = oracle.quant_int8(x, 64, 16)
    c1, s1 = oracle.quant_int8(x * np.float32(8.0), 64, 16)
    assert np.array_equal(c0, c1) and np.array_equal(s1, s0 * np.float32(8.0))
    # changing one group's values leaves the other groups untouched
    y = x.copy()
    y[16:32] *= np.float32(3.7)
    c2, s2 = oracle.quant_int8(y, 64, 16)
    keep = np.r_[0:16, 32:64]
    assert np.array_equal(c2[keep], c0[keep]) and s2[0] == s0[0] and np.array_equal(s2[2:], s0[2:])
    # each group's largest magnitude maps to +-127
    for g in range(4):
        blk = c0[g * 16:(g + 1) * 16]
        assert np.abs(blk.astype(np.int32)).max() == 127


def test_int8_tail_group_and_padding_rows():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((40, 8)).astype(np.float32)
    x[37:] = 1e3                       # rows past n_valid must be ignored
    c, s = oracle.quant_int8(x, 37, 16)
    assert s.shape == (3,)
    assert np.all(c[37:] == 0)
    tail = x[32:37]
    assert s[2] == np.float32(np.abs(tail).max()) / np.float32(127)


def test_v_fp8_per_channel():
    rng = np.random.default_rng(14)
    v = (rng.standard_normal((50, 16)) * np.linspace(0.1, 9, 16)).astype(np.float32)
    v[:, 3] = 0.0
    codes, sc = oracle.quant_v_fp8(v)
    amax = np.abs(v).max(axis=0)
    assert sc[3] == 0 and np.all(codes[:, 3] == 0)
    nz = amax > 0
    assert np.array_equal(sc[nz], amax[nz] / np.float32(448))
    inv = np.float32(448) / amax[nz]
    t = np.clip(v[:, nz] * inv[None, :], -448, 448).astype(np.float32)
    ref = torch.from_numpy(np.ascontiguousarray(t)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[:, nz], ref)
    # each channel's largest magnitude maps to +-448 (code 0x7e / 0xfe)
    for c in np.nonzero(nz)[0]:
        assert (codes[:, c] & 0x7F).max() == 0x7E


def test_exact_mean_is_correctly_rounded():
    rng = np.random.default_rng(15)
    for dt in (np.float16, "bf16"):
        x = (rng.standard_normal((300, 5)) * rng.uniform(0.001, 100, 5)).astype(np.float32)
        if dt == "bf16":
            x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
        else:
            x = x.astype(np.float16).astype(np.float32)
        m = oracle.exact_mean(x)
        for c in range(5):
            exact = sum((Fraction(float(t)) for t in x[:, c]), Fraction(0))
            s64 = float(exact)                      # correctly rounded to fp64
            assert m[c] == np.float32(s64 / 300)
        # order independence
        perm = rng.permutation(300)
        assert np.array_equal(oracle.exact_mean(x[perm]), m)


def test_exact_mean_cancellation():
    # values whose naive float32 running sum loses the small terms
    x = np.array([[65504.0], [1.0], [-65504.0], [2.0 ** -24]] * 3, dtype=np.float32)
    m = oracle.exact_mean(x)
    assert m[0] == np.float32((3 * (1.0 + 2.0 ** -24)) / 12)


def test_reference_forward_smoothing_and_layouts():
    """K' = fl32(K - mean) before quantization; HND and NHD give identical results."""
    rng = np.random.default_rng(16)
    q = rng.standard_normal((1, 2, 70, 40)).astype(np.float16).astype(np.float32)
    k = (rng.standard_normal((1, 2, 70, 40)) + 3.0).astype(np.float16).astype(np.float32)
    v = rng.standard_normal((1, 2, 70, 40)).astype(np.float16).astype(np.float32)
    r = oracle.reference_forward(q, k, v, dtype="fp16", layout="HND", gran="per_thread", attention=False)
    km = r["k_mean"][0][0]
    assert km.shape == (64,) and np.all(km[40:] == 0)
    kp = np.zeros((70, 64), np.float32)
    kp[:, :40] = k[0, 0] - km[None, :40]
    c, s = oracle.quant_int8(kp, 70, 16)
    assert np.array_equal(r["k8"][0][0], c) and np.array_equal(r["k_scale"][0][0], s)
    r2 = oracle.reference_forward(q.transpose(0, 2, 1, 3).copy(), k.transpose(0, 2, 1, 3).copy(),
                                  v.transpose(0, 2, 1, 3).copy(), dtype="fp16", layout="NHD",
                                  gran="per_thread", attention=False)
    for key in ("q8", "q_scale", "k8", "k_scale", "k_mean", "v8", "v_scale"):
        assert np.array_equal(r[key][0], r2[key][0]), key
