"""Pins of the oracle's attention steps.

* The fp64 exact mode is checked against a NumPy/SciPy brute-force softmax
  attention and against the softmax invariants (rows of P sum to one, the
  output is unchanged when every score of a row shifts by the same amount --
  the property smooth_k relies on -- and causal masking hides future keys).
* The quantized (emulated) mode is checked against exact attention evaluated
  on its own dequantized operands, within the error bound that rounding P to
  fp16 or FP8 allows; against the closed form of the FlashAttention-style
  update over many key tiles (cumulative maximum, torch's float8/fp16 casts),
  which fixes the reference maximum and every P operand bit for bit; against
  the convex-combination property of the normalised quantized weights;
  against exact integer score dumps and the closed-form log-sum-exp; and the
  rounding allowance against perturbed evaluations.

Sources: SageAttention deployment guide (pwwt.cn), sec. 1 (softmax(QK^T)V with
INT8 Q/K and FP8 V), sec. 4.1 (sm_scale default 1/sqrt(head_dim), is_causal,
return_lse), sec. 4.2 (smooth_k); SageAttention 2.2.0 on the RX 9070 XT
(pnsm.cn), sec. 2 (blockwise softmax as in FlashAttention).
"""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle


def _half(shape, rng, scale=1.0, bias=0.0):
    return (rng.standard_normal(shape) * scale + bias).astype(np.float16).astype(np.float32)


def _brute(q, k, v, sm, causal):
    s = (q.astype(np.float64) @ k.astype(np.float64).T) * sm
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= np.arange(q.shape[0])[:, None], s, -np.inf)
    p = sps.softmax(s, axis=1)
    return p @ v.astype(np.float64), sps.logsumexp(s, axis=1)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,d", [(37, 37, 16), (20, 75, 40), (64, 33, 128)])
def test_exact_mode_matches_bruteforce(causal, nq, nk, d):
    rng = np.random.default_rng(nq * 7 + nk + d)
    q, k, v = _half((1, 2, nq, d), rng), _half((1, 2, nk, d), rng), _half((1, 2, nk, d), rng)
    r = oracle.exact_forward(q, k, v, layout="HND", causal=causal)
    for h in range(2):
        o, l = _brute(q[0, h], k[0, h], v[0, h], 1 / math.sqrt(d), causal)
        assert np.max(np.abs(r["out"][0][h] - o)) < 1e-12
        assert np.max(np.abs(r["lse"][0][h] - l)) < 1e-12


def test_exact_mode_invariants():
    rng = np.random.default_rng(3)
    nq, nk, d = 48, 80, 64
    q, k, v = _half((1, 1, nq, d), rng), _half((1, 1, nk, d), rng), _half((1, 1, nk, d), rng)
    # rows of P sum to one: V = 1 gives out = 1
    r1 = oracle.exact_forward(q, k, np.ones_like(v), causal=True)
    assert np.max(np.abs(r1["out"][0] - 1.0)) < 1e-13
    # a per-channel shift of K shifts every score of a row by q_i.delta:
    # the output is unchanged and lse moves by sm_scale * q_i.delta
    delta = rng.standard_normal(d).astype(np.float64) * 3
    r0 = oracle.exact_forward(q, k, v)
    k2 = k.astype(np.float64) + delta[None, None, None, :]
    r2 = oracle.exact_forward(q.astype(np.float64), k2, v.astype(np.float64))
    assert np.max(np.abs(r2["out"][0] - r0["out"][0])) < 1e-12
    corr = (q[0, 0].astype(np.float64) @ delta) / math.sqrt(d)
    assert np.max(np.abs(r2["lse"][0][0] - r0["lse"][0][0] - corr)) < 1e-11
    # causal: perturbing keys/values after row i leaves row i unchanged
    rc = oracle.exact_forward(q, k, v, causal=True)
    kp, vp = k.copy(), v.copy()
    kp[:, :, 30:] += 5.0
    vp[:, :, 30:] -= 7.0
    rp = oracle.exact_forward(q, kp, vp, causal=True)
    assert np.array_equal(rc["out"][0][:, :30], rp["out"][0][:, :30])
    assert not np.allclose(rc["out"][0][:, 30:], rp["out"][0][:, 30:])


def _dequantized(r, b, h, hk, gran, v_dtype, dtype):
    """q_hat = q8 * qscale, k_hat = k8 * kscale (smoothed K), v_hat = operand
    values with the V scale and mean applied."""
    gq, gk = oracle.Q_GROUP[gran], oracle.K_GROUP[gran]
    q8, k8 = r["q8"][b][h].astype(np.float64), r["k8"][b][hk].astype(np.float64)
    qs = np.repeat(r["q_scale"][b][h], gq)[:q8.shape[0]].astype(np.float64)
    ks = np.repeat(r["k_scale"][b][hk], gk)[:k8.shape[0]].astype(np.float64)
    if v_dtype == "fp8":
        vv = oracle.e4m3_decode(r["v8"][b][hk]).astype(np.float64) * r["v_scale"][b][hk][None, :]
    else:
        vv = r["v16"][b][hk].astype(np.float64)
    return q8 * qs[:, None], k8 * ks[:, None], vv, r["v_mean"][b][hk].astype(np.float64)


@pytest.mark.parametrize("gran", ["per_block", "per_warp", "per_thread"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp16_path_matches_exact_on_dequantized(gran, causal):
    """With P rounded to fp16 the emulation differs from exact attention on its
    own dequantized operands only by that rounding: P = p (1 + d) with
    |d| <= 2^-11 for normal p (plus 2^-25 absolute below the fp16 normal
    range), and the weights P_j / sum P differ from p_j / sum p by at most a
    factor (1 +- 2^-11) / (1 -+ 2^-11), so
    |out - out_exact| <= (2^-10 + n_k 2^-24) max|v| (l >= 1)."""
    rng = np.random.default_rng(21)
    nq, nk, d = 150, 200, 48
    q = _half((1, 3, nq, d), rng)
    k = _half((1, 3, nk, d), rng, bias=0.7)
    v = _half((1, 3, nk, d), rng, bias=-0.3)
    r = oracle.reference_forward(q, k, v, dtype="fp16", gran=gran, v_dtype="fp16", smooth_k=True,
                                 smooth_v=True, causal=causal, bk=64)
    for h in range(3):
        qh, kh, vh, vm = _dequantized(r, 0, h, h, gran, "fp16", "fp16")
        vfull = vh + vm[None, :]
        ex = oracle.exact_forward(qh[None, None], kh[None, None], vfull[None, None], causal=causal,
                                  sm_scale=1 / math.sqrt(d))
        bound = (2.0 ** -10 * (1 + 2.0 ** -10) + nk * 2.0 ** -24) * np.abs(vh).max() + 1e-6
        err = np.abs(r["out"][0][h] - ex["out"][0][0][:, :d]).max()
        assert err <= bound, (err, bound)


LOG2E32 = np.float32(1.4426950408889634)


def _closed_form(r, b, h, hk, gran, sm, causal, bk=64, v_dtype="fp8", dtype="fp16", pp_factor=None,
                 want_l=False):
    """The FlashAttention-style online softmax written in closed form instead
    of as a loop: with m_t the running maximum after key tile t (a cumulative
    maximum of the tile maxima), every key j of tile t gets the operand
    P_j = Q(fl32(fl32(2^fl32(s_j - m_t)) * Pscale)) and the weight
    P_j 2^(m_t - m_T) at the final maximum m_T, and
    out = sum_j w_j v_j / sum_j w_j.  Scores and exponents use NumPy float32
    arithmetic (one rounding per operation), Q is torch's float8_e4m3fn or
    fp16/bf16 cast.  pp_factor (nq, nk), if given, multiplies the value
    before the operand rounding (an evaluation with a different exponent).
    Returns P (nq, nk), m_t per key (nq, nk), out (nq, d) in fp64 and, with
    want_l, also l (nq,), the sum of the weights at the final maximum."""
    gq, gk = oracle.Q_GROUP[gran], oracle.K_GROUP[gran]
    q8 = r["q8"][b][h].astype(np.int64)
    k8 = r["k8"][b][hk].astype(np.int64)
    nq, nk = q8.shape[0], k8.shape[0]
    S = q8 @ k8.T
    assert np.abs(S).max() < 2 ** 24
    qs = np.repeat(r["q_scale"][b][h], gq)[:nq].astype(np.float32)
    ks = np.repeat(r["k_scale"][b][hk], gk)[:nk].astype(np.float32)
    c = (qs * np.float32(sm)) * LOG2E32
    s = (S.astype(np.float32) * ks[None, :]) * c[:, None]
    vis = np.ones((nq, nk), bool)
    if causal:
        vis = np.arange(nk)[None, :] <= np.arange(nq)[:, None]
    sv = np.where(vis, s, np.float32(-np.inf))
    nt = -(-nk // bk)
    tm = np.full((nq, nt), -np.inf, np.float32)
    for t in range(nt):
        tm[:, t] = sv[:, t * bk:(t + 1) * bk].max(axis=1)
    mt = np.maximum.accumulate(tm, axis=1)
    m_key = np.repeat(mt, bk, axis=1)[:, :nk]
    x = np.where(vis, s - m_key, np.float32(-np.inf)).astype(np.float32)
    p = np.exp2(x.astype(np.float64)).astype(np.float32)
    pscale = 448.0 if v_dtype == "fp8" else 1.0
    pp = (p.astype(np.float64) * pscale).astype(np.float32)
    if pp_factor is not None:
        pp = (pp.astype(np.float64) * pp_factor).astype(np.float32)
    if v_dtype == "fp8":
        P = torch.from_numpy(np.minimum(pp, 448.0)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        vv = oracle.e4m3_decode(r["v8"][b][hk]).astype(np.float64)
        vsc = r["v_scale"][b][hk].astype(np.float64)
    else:
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        P = torch.from_numpy(pp).to(tdt).to(torch.float64).numpy()
        vv = r["v16"][b][hk].astype(np.float64)
        vsc = np.ones(vv.shape[1])
    P = np.where(vis, P, 0.0)
    mfin = mt[:, -1:].astype(np.float64)
    w = P * np.exp2(m_key.astype(np.float64) - mfin)
    w = np.where(vis, w, 0.0)
    out = (w @ vv) / w.sum(axis=1, keepdims=True) * vsc[None, :] + r["v_mean"][b][hk].astype(np.float64)[None, :]
    if want_l:
        return P, np.where(vis, m_key, np.float32(-np.inf)), out, w.sum(axis=1)
    return P, np.where(vis, m_key, np.float32(-np.inf)), out


@pytest.mark.parametrize("gran,causal,v_dtype,dtype", [("per_warp", False, "fp8", "fp16"),
                                                       ("per_thread", True, "fp8", "bf16"),
                                                       ("per_block", False, "fp16", "fp16"),
                                                       ("per_thread", True, "fp16", "bf16")])
def test_multi_tile_closed_form(gran, causal, v_dtype, dtype):
    """Over many key tiles the oracle's online softmax equals the closed form
    above: the same reference maximum for every key (the plain update
    m' = max(m, tile max); a lazy update that keeps m until a tile exceeds it
    by a margin fails), the same P operand codes bit for bit (the exponent
    fl32(s - m') and P's scale 448; any other exponent formation moves some
    codes), and the same outputs to fp64 rounding."""
    rng = np.random.default_rng(40)
    nq, nk, d = (300, 300, 64) if causal else (70, 700, 64)
    q = _half((1, 2, nq, d), rng, scale=1.5)
    k = _half((1, 2, nk, d), rng, bias=0.4)
    v = _half((1, 2, nk, d), rng)
    r = oracle.reference_forward(q, k, v, dtype=dtype, gran=gran, v_dtype=v_dtype, causal=causal, smooth_v=True,
                                 want_p=True)
    for h in range(2):
        P, mref, out = _closed_form(r, 0, h, h, gran, 1 / math.sqrt(d), causal, v_dtype=v_dtype, dtype=dtype)
        np.testing.assert_array_equal(r["mref"][0][h], mref)
        np.testing.assert_array_equal(r["p"][0][h], P)
        assert np.max(np.abs(r["out"][0][h] - out)) <= 1e-12 * max(1.0, np.abs(out).max())
        # the maximum really moves over the tiles, so the rescaling is exercised
        mt = mref[:, ::64].astype(np.float64)
        steps = np.diff(np.where(np.isfinite(mt), mt, np.nan), axis=1)
        assert np.nansum(steps > 0) > nq / 2


def test_quantized_weights_form_a_convex_combination():
    """The normaliser is the sum of the quantized P that multiply V: with V
    constant along the sequence (an E4M3 value times its scale) the output is
    that constant to fp64 rounding, for any scores, and the weights
    P_j 2^(m_t - m_T) divided by their sum reproduce every output.  A
    normaliser summing the unrounded p would miss by up to the FP8 rounding of
    P (a few per cent)."""
    rng = np.random.default_rng(41)
    nq, nk, d = 40, 333, 64
    q = _half((1, 1, nq, d), rng, scale=2.0)
    k = _half((1, 1, nk, d), rng)
    col = rng.standard_normal(d).astype(np.float16).astype(np.float32)
    v = np.broadcast_to(col[None, None, None, :], (1, 1, nk, d)).copy()
    for causal in (False, True):
        r = oracle.reference_forward(q, k, v, dtype="fp16", gran="per_thread", causal=causal, smooth_v=False,
                                     want_p=True)
        # every key has the same V codes, so the dequantized V is one row repeated
        vdec = oracle.e4m3_decode(r["v8"][0][0]).astype(np.float64) * r["v_scale"][0][0][None, :]
        assert np.array_equal(vdec, np.broadcast_to(vdec[0], vdec.shape))
        assert np.max(np.abs(r["out"][0][0] - vdec[0][None, :])) <= 1e-13
        assert np.max(np.abs(vdec[0] - col)) <= 2.0 ** -4 * np.abs(col).max()
        P, mref = r["p"][0][0], r["mref"][0][0].astype(np.float64)
        mfin = np.max(mref, axis=1, keepdims=True)
        w = np.where(np.isfinite(mref), P * np.exp2(np.where(np.isfinite(mref), mref, 0.0) - mfin), 0.0)
        # the dumped weights, normalised by their own sum, reproduce the output
        # with a non-constant V as well
        v2 = _half((1, 1, nk, d), rng)
        r2 = oracle.reference_forward(q, k, v2, dtype="fp16", gran="per_thread", causal=causal, want_p=True)
        assert np.array_equal(r2["p"][0][0], P)
        v2dec = oracle.e4m3_decode(r2["v8"][0][0]).astype(np.float64) * r2["v_scale"][0][0][None, :]
        o2 = (w / w.sum(axis=1, keepdims=True)) @ v2dec
        assert np.max(np.abs(o2 - r2["out"][0][0])) <= 1e-12


def test_causal_p_structure():
    """Causal rows give zero P (and no reference maximum) to keys after the
    row; key 0 is always seen, and the largest operand of a row is 448 at
    the key where the row's running maximum was set."""
    rng = np.random.default_rng(42)
    nq, nk, d = 150, 150, 64
    q, k, v = _half((1, 1, nq, d), rng), _half((1, 1, nk, d), rng), _half((1, 1, nk, d), rng)
    r = oracle.reference_forward(q, k, v, dtype="fp16", gran="per_thread", causal=True, want_p=True)
    P, mref = r["p"][0][0], r["mref"][0][0]
    future = np.arange(nk)[None, :] > np.arange(nq)[:, None]
    assert np.all(P[future] == 0.0) and np.all(np.isneginf(mref[future]))
    assert np.all(P[:, 0] > 0.0) or np.all(np.isfinite(mref[:, 0]))
    assert np.all(P.max(axis=1) == 448.0)


@pytest.mark.parametrize("v_dtype,dtype", [("fp8", "fp16"), ("fp16", "bf16")])
def test_allowance_bounds_a_perturbed_evaluation(v_dtype, dtype):
    """The allowance is what it claims: an evaluation whose values before the
    P rounding differ from the oracle's by factors within 2^(+-delta_ij)
    (delta from exp_band) lands within the allowance of the oracle's output.
    A wide band makes many operands change."""
    rng = np.random.default_rng(43)
    nq, nk, d = 50, 500, 64
    q, k, v = _half((1, 1, nq, d), rng, scale=1.5), _half((1, 1, nk, d), rng), _half((1, 1, nk, d), rng)
    band = (40.0, 2.0 ** -12)
    r = oracle.reference_forward(q, k, v, dtype=dtype, gran="per_warp", v_dtype=v_dtype, smooth_v=True,
                                 exp_band=band, want_p=True)
    z = oracle.reference_forward(q, k, v, dtype=dtype, gran="per_warp", v_dtype=v_dtype, smooth_v=True)
    assert np.all(z["allow"][0] == 0.0)
    assert np.array_equal(z["out"][0], r["out"][0])
    # delta per (row, key) from the same quantities the oracle uses
    qs = np.repeat(r["q_scale"][0][0], 32)[:nq].astype(np.float32)
    ks = np.repeat(r["k_scale"][0][0], 64)[:nk].astype(np.float32)
    c = (qs * np.float32(1 / math.sqrt(d))) * LOG2E32
    S = r["q8"][0][0].astype(np.int64) @ r["k8"][0][0].astype(np.int64).T
    s = (S.astype(np.float32) * ks[None, :]) * c[:, None]
    mref = r["mref"][0][0].astype(np.float64)
    delta = band[0] * c.astype(np.float64)[:, None] * ks.astype(np.float64)[None, :] + \
        band[1] * (np.abs(s.astype(np.float64)) + np.abs(mref) + 8.0)
    _, _, _, l0 = _closed_form(r, 0, 0, 0, "per_warp", 1 / math.sqrt(d), False, v_dtype=v_dtype, dtype=dtype,
                               want_l=True)
    moved = 0
    for trial in range(4):
        u = rng.uniform(-1.0, 1.0, size=(nq, nk)) if trial else np.sign(rng.uniform(-1, 1, size=(nq, nk)))
        fac = np.exp2(0.999 * u * delta)
        P2, _, out2, l2 = _closed_form(r, 0, 0, 0, "per_warp", 1 / math.sqrt(d), False, v_dtype=v_dtype,
                                       dtype=dtype, pp_factor=fac, want_l=True)
        moved += int((P2 != r["p"][0][0]).sum())
        assert np.all(np.abs(out2 - r["out"][0][0]) <= r["allow"][0][0] + 1e-12)
        # the log-sum-exp moves with ln l
        assert np.all(np.abs(np.log(l2) - np.log(l0)) <= r["lse_allow"][0][0] + 1e-12)
    assert moved > 100 and r["allow"][0][0].max() > 0 and r["lse_allow"][0][0].max() > 0
    assert np.all(z["lse_allow"][0] == 0.0)


def test_fp8_schedule_without_max_updates_equals_single_tile():
    """If every row's maximum lies in the first key tile, later tiles never
    move the reference maximum, so a 16-key schedule reproduces the one-tile
    result exactly (up to fp64 summation order)."""
    rng = np.random.default_rng(23)
    nq, nk, d = 32, 96, 64
    q = np.abs(_half((1, 1, nq, d), rng))
    k = _half((1, 1, nk, d), rng)
    k[0, 0, :16] = np.abs(k[0, 0, :16]) + 2.0      # first tile dominates every row
    v = _half((1, 1, nk, d), rng)
    a = oracle.reference_forward(q, k, v, dtype="fp16", gran="per_thread", smooth_k=False, bk=16)
    b = oracle.reference_forward(q, k, v, dtype="fp16", gran="per_thread", smooth_k=False, bk=96)
    assert np.max(np.abs(a["out"][0] - b["out"][0])) < 1e-12
    # with the maximum in the last tile the schedules differ (P8 rounds at
    # different reference maxima) but both stay within the FP8 bound
    k2 = k.copy()
    k2[0, 0, :16] = _half((16, d), rng)
    k2[0, 0, 80:] = np.abs(k2[0, 0, 80:]) + 2.0
    a2 = oracle.reference_forward(q, k2, v, dtype="fp16", gran="per_thread", smooth_k=False, bk=16)
    b2 = oracle.reference_forward(q, k2, v, dtype="fp16", gran="per_thread", smooth_k=False, bk=96)
    d2 = np.abs(a2["out"][0] - b2["out"][0])
    assert d2.max() > 1e-9 and d2.max() < 2 * 2.0 ** -4 * np.abs(v).max()


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_path_within_bound_and_scores_exact(causal):
    """E4M3 rounding of P (scaled to 448 / 2^tau) has relative error <= 2^-4
    for normal values and absolute error <= 2^-10 below 2^-6; normalising by
    the sum of the rounded P gives
    |out - out_exact| <= (2^-3 / (1 - 2^-4) + n_k 2^-9 2^tau / 448) max|v_hat|."""
    rng = np.random.default_rng(24)
    nq, nk, d = 130, 190, 128
    q, k, v = _half((2, 2, nq, d), rng), _half((2, 2, nk, d), rng, bias=0.5), _half((2, 2, nk, d), rng)
    r = oracle.reference_forward(q, k, v, dtype="fp16", gran="per_thread", v_dtype="fp8", causal=causal,
                                 want_scores=True, smooth_v=True)
    for b in range(2):
        for h in range(2):
            S = r["q8"][b][h].astype(np.int64) @ r["k8"][b][h].astype(np.int64).T
            assert np.array_equal(r["scores"][b][h], S)
            qh, kh, vh, vm = _dequantized(r, b, h, h, "per_thread", "fp8", "fp16")
            ex = oracle.exact_forward(qh[None, None], kh[None, None], (vh + vm[None, :])[None, None],
                                      causal=causal, sm_scale=1 / math.sqrt(d))
            bound = (2.0 ** -3 / (1 - 2.0 ** -4) + nk * 2.0 ** -9 / 448) * np.abs(vh).max()
            err = np.abs(r["out"][b][h] - ex["out"][0][0]).max()
            assert err <= bound, (err, bound)
            # typical error is far below the worst-case bound
            assert np.sqrt(np.mean((r["out"][b][h] - ex["out"][0][0]) ** 2)) < 0.05 * bound


def test_lse_closed_form_with_smoothing():
    """lse is the log-sum-exp of the unsmoothed dequantized scores,
    ln sum_j exp(sm_scale q_hat_i.(k_hat'_j + mean_k)), up to the rounding of
    the P values that l sums: within ln(1 + 2^-11) on the fp16 path."""
    rng = np.random.default_rng(25)
    nq, nk, d = 64, 150, 64
    q, k, v = _half((1, 2, nq, d), rng), _half((1, 2, nk, d), rng, bias=1.5), _half((1, 2, nk, d), rng)
    for causal in (False, True):
        r = oracle.reference_forward(q, k, v, dtype="fp16", gran="per_warp", smooth_k=True, causal=causal,
                                     v_dtype="fp16")
        for h in range(2):
            qh, kh, _, _ = _dequantized(r, 0, h, h, "per_warp", "fp16", "fp16")
            km = r["k_mean"][0][h].astype(np.float64)
            s = (qh @ (kh + km[None, :]).T) / math.sqrt(d)
            if causal:
                s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, -np.inf)
            ref = sps.logsumexp(s, axis=1)
            assert np.max(np.abs(r["lse"][0][h] - ref)) < 2.0 ** -10


def test_gqa_and_varlen_slicing():
    """GQA uses K/V head h // (Hq/Hkv); a packed varlen batch equals separate
    dense problems (means, groups and scales restart per sequence)."""
    rng = np.random.default_rng(26)
    lens = [70, 33, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = _half((T, 4, 64), rng), _half((T, 2, 64), rng, bias=1.0), _half((T, 2, 64), rng)
    r = oracle.reference_forward(q, k, v, dtype="fp16", cu_seqlens_q=cu, cu_seqlens_k=cu, causal=True,
                                 gran="per_thread")
    for b, n in enumerate(lens):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        qb = q[sl].transpose(1, 0, 2)[None].copy()
        kb = np.repeat(k[sl].transpose(1, 0, 2), 2, axis=0)[None].copy()
        vb = np.repeat(v[sl].transpose(1, 0, 2), 2, axis=0)[None].copy()
        rb = oracle.reference_forward(qb, kb, vb, dtype="fp16", causal=True, gran="per_thread")
        assert np.array_equal(r["out"][b], rb["out"][0])
        assert np.array_equal(r["q8"][b], rb["q8"][0])
        assert np.array_equal(r["k8"][b], rb["k8"][0][::2])


def test_lse_pq_share_of_p_rounding():
    """lse_pq is |ln sum(rounded P) - ln sum(P)|: 0 when every P is exactly
    representable, and within the format's relative rounding bound
    (2^-4 for E4M3 normals, 2^-11 for fp16) otherwise."""
    rng = np.random.default_rng(31)
    k = _half((1, 1, 150, 64), rng)
    v = _half((1, 1, 150, 64), rng)
    # Q = 0: every score is 0, so every P is 448 (p = 1 at the maximum), an E4M3 value
    r0 = oracle.reference_forward(np.zeros((1, 1, 40, 64), np.float32), k, v, dtype="fp16", gran="per_thread")
    assert np.all(r0["lse_pq"][0] == 0.0)
    q = _half((1, 1, 40, 64), rng, scale=2.0)
    r8 = oracle.reference_forward(q, k, v, dtype="fp16", gran="per_thread")
    pq8 = r8["lse_pq"][0]
    assert np.all(pq8 > 0) and np.all(pq8 <= -math.log1p(-2.0 ** -4))
    r16 = oracle.reference_forward(q, k, v, dtype="fp16", gran="per_thread", v_dtype="fp16")
    pq16 = r16["lse_pq"][0]
    assert np.all(pq16 <= -math.log1p(-2.0 ** -11)) and pq16.max() < pq8.max()
