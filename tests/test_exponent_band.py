"""The exponent band of the parity tolerance, checked by evaluating both
exponent forms on the CPU.

The kernel forms the log2 of P's value before its operand rounding as
x_k = fl32((B + S) f + fl32(nb - B f)), nb = fl32(fl32(log2 448) - m'),
with B + S exact (B < 2^24 is the integer the score accumulator starts from,
read as a float) and f = fl32(kscale c_i), then takes v_exp_f32 (1 ulp).  The
oracle forms x = fl32(s - m'), s = fl32(fl32(S kscale) c_i), p = fl32(2^x),
P_pre = fl32(p * 448).  The tolerance assumes the two values of P before the
operand rounding differ by a factor within 2^(+-delta),
delta = f + 2^-21 (|s| + |m'| + 8) (EXP_BAND in parity_utils).  Here both
forms are evaluated with NumPy float32 arithmetic (fused multiply-adds
emulated in fp64, exact for these operand widths before the final rounding)
over scale factors and scores spanning the ranges the quantizers produce,
with each side's maximum taken from its own score form, and 1 ulp allowed for
each exponential.
"""
import math

import numpy as np

from parity_utils import EXP_BAND

B = float(2 ** 23 + 0x22F983)          # any bias in [2^23, 2^24) with B + S exact behaves alike
L8 = np.float32(math.log2(448.0))
LOG2E = np.float32(1.4426950408889634)


def _fma32(a, b, c):
    """fl32(a * b + c) with a single rounding (a, b, c float32; the fp64 product
    of two float32 values is exact and the fp64 sum is within 2^-53 relative)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def test_band_covers_both_exponent_forms():
    rng = np.random.default_rng(50)
    n = 400_000
    worst = 0.0
    for trial in range(8):
        # scale factors over many binades, scores up to the INT8 limit 128 * 127^2
        qs = np.exp2(rng.uniform(-12, 6, n)).astype(np.float32)
        ks = np.exp2(rng.uniform(-12, 6, n)).astype(np.float32)
        sm = np.float32(1 / math.sqrt(rng.choice([16, 64, 96, 128])))
        smax = 2064512 if trial % 2 else 300000
        S = rng.integers(-smax, smax + 1, n)
        S_row_max = np.minimum(S + rng.integers(0, 200000, n), smax)
        ci = (qs * sm) * LOG2E
        # oracle form
        s_o = (S.astype(np.float32) * ks) * ci
        m_o = (S_row_max.astype(np.float32) * ks) * ci
        x_o = np.minimum(s_o - m_o, np.float32(0.0))
        ok = s_o <= m_o
        p_o = np.exp2(x_o.astype(np.float64)).astype(np.float32)
        pp_o = (p_o.astype(np.float64) * 448.0).astype(np.float32)
        # kernel form
        f = ks * ci
        s_k = S.astype(np.float32) * f
        m_k = S_row_max.astype(np.float32) * f
        nb = L8 - m_k
        c = _fma32(np.full(n, -B, np.float32), f, nb)
        x_k = _fma32((B + S).astype(np.float32), f, c)
        # log2 of each side's value before the operand rounding, with 1 ulp for
        # the kernel's exp2 (the oracle's fp32 rounding of 2^x is inside pp_o)
        keep = ok & (pp_o > 2.0 ** -12) & np.isfinite(x_k)
        lo = np.log2(pp_o[keep].astype(np.float64))
        kx = x_k[keep].astype(np.float64)
        diff = np.abs(lo - kx) + 2.0 ** -23 / math.log(2)
        delta = EXP_BAND[0] * (ci[keep].astype(np.float64) * ks[keep].astype(np.float64)) + \
            EXP_BAND[1] * (np.abs(s_o[keep].astype(np.float64)) + np.abs(m_o[keep].astype(np.float64)) + 8.0)
        assert np.all(diff <= delta), (diff / delta).max()
        worst = max(worst, float((diff / delta).max()))
    # the band is not loose by orders of magnitude either
    assert worst > 0.05
