"""CPU oracle for the quantized attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and it imports nothing from the product
path: the two share no code.  The seeded input generators live in
``workloads.py``, which holds none of the method's arithmetic.

The arithmetic lives in ``sage_oracle.c`` (plain loops, fp32 quantization
decisions, fp64 accumulation) plus the exact per-channel means below.  This
module slices the caller's tensor layout into per-(sequence, head) problems,
runs the method's steps in the pages' order, and returns every intermediate
that the GPU path exposes.

Sources, cited by title and section:
  [guide]    SageAttention deployment guide (pwwt.cn/news/4103508)
  [amd-9070] SageAttention 2.2.0 on the RX 9070 XT (pnsm.cn/news/1834815)

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library routines and brute force on tiny inputs (see
those tests); no function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Callable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsage_oracle.so")
# the oracle's own mutation tests load deliberately broken builds from here
_LIB_OVERRIDE = os.environ.get("SAGE_ORACLE_LIB")

# key/query group sizes per granularity (reading of [guide] sec. 4.2,
# qk_quant_gran; per_thread is the finest): rows of Q sharing one scale and
# keys of K sharing one scale.
Q_GROUP = {"per_block": 128, "per_warp": 32, "per_thread": 1}
K_GROUP = {"per_block": 64, "per_warp": 64, "per_thread": 16}

# key tile of the online softmax (keys per block of the FlashAttention-style
# update; see oracle_attn_rows in sage_oracle.c)
DEFAULT_BK = 64


def build(force: bool = False) -> str:
    """Compile the oracle library with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               _SRC, "-o", _LIB_PATH, "-lm"]
        subprocess.check_call(cmd)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_float
        L.oracle_round_half.argtypes = [ctypes.c_float, i]
        L.oracle_round_half.restype = ctypes.c_float
        L.oracle_e4m3_encode_array.argtypes = [P, ctypes.c_int64, P]
        L.oracle_e4m3_encode_array.restype = None
        L.oracle_round_half_array.argtypes = [P, ctypes.c_int64, i, P]
        L.oracle_round_half_array.restype = None
        L.oracle_quant_int8_rows.argtypes = [P, i, i, i, i, P, P]
        L.oracle_quant_int8_rows.restype = None
        L.oracle_quant_v_fp8.argtypes = [P, i, i, P, P]
        L.oracle_quant_v_fp8.restype = None
        d_ = ctypes.c_double
        L.oracle_attn_rows.argtypes = [i, i, i, P, P, P, P, P, P, P, P, ctypes.c_float, i, i, i, i, d_, d_,
                                       i, P, P, P, P, P, P, P, P, P]
        L.oracle_attn_rows.restype = i
        L.oracle_attn_exact.argtypes = [i, i, i, P, P, P, ctypes.c_double, i, i, i, P, P, P]
        L.oracle_attn_exact.restype = i
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------- codecs
def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 -> E4M3FN code bytes (clamped to +-448, round to nearest even)."""
    flat = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    out = np.zeros(flat.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_p(flat), flat.size, _p(out))
    return out.reshape(np.shape(x))


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    L = lib()
    table = np.array([L.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float32)
    return table[np.asarray(codes, dtype=np.uint8)]


def round_half(x: np.ndarray, dtype: str) -> np.ndarray:
    flat = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    out = np.zeros(flat.shape, dtype=np.float32)
    lib().oracle_round_half_array(_p(flat), flat.size, 1 if dtype == "bf16" else 0, _p(out))
    return out.reshape(np.shape(x))


# --------------------------------------------------------------------------- steps
def padded_head_dim(d: int) -> int:
    """Head dim padding ([guide] sec. 4.1): d < 64 is zero-padded to 64,
    64 < d < 128 to 128, d > 128 is an error."""
    if d <= 0 or d > 128:
        raise ValueError(f"head_dim {d} unsupported (1..128)")
    return 64 if d <= 64 else 128


def exact_mean(x: np.ndarray) -> np.ndarray:
    """Per-channel mean along the sequence ([guide] sec. 4.2, smooth_k /
    smooth_v).  Reading: fl32(fl64(exact sum) / N); math.fsum returns the
    correctly rounded sum, so the result is independent of summation order.
    x: (N, D) float32 holding exact fp16/bf16 values."""
    n = x.shape[0]
    out = np.zeros(x.shape[1], dtype=np.float32)
    if n == 0:
        return out
    for c in range(x.shape[1]):
        out[c] = np.float32(math.fsum(x[:, c].tolist()) / n)
    return out


def quant_int8(x: np.ndarray, n_valid: int, group: int):
    """INT8 group quantization of an (N, Dp) fp32 matrix; see sage_oracle.c."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, dp = x.shape
    codes = np.zeros((rows, dp), dtype=np.int8)
    scales = np.zeros((rows + group - 1) // group, dtype=np.float32)
    lib().oracle_quant_int8_rows(_p(x), rows, n_valid, dp, group, _p(codes), _p(scales))
    return codes, scales


def quant_v_fp8(v: np.ndarray):
    v = np.ascontiguousarray(v, dtype=np.float32)
    n, dp = v.shape
    codes = np.zeros((n, dp), dtype=np.uint8)
    scales = np.zeros(dp, dtype=np.float32)
    lib().oracle_quant_v_fp8(_p(v), n, dp, _p(codes), _p(scales))
    return codes, scales


def _problems(x: np.ndarray, layout: str, cu: Optional[np.ndarray]):
    """Yield (b, array (H, N_b, D)) per sequence from the caller's layout."""
    if cu is not None:
        for b in range(len(cu) - 1):
            yield b, x[int(cu[b]):int(cu[b + 1])].transpose(1, 0, 2)
    elif layout == "HND":
        for b in range(x.shape[0]):
            yield b, x[b]
    elif layout == "NHD":
        for b in range(x.shape[0]):
            yield b, x[b].transpose(1, 0, 2)
    else:
        raise ValueError(layout)


def _pad(x: np.ndarray, dp: int) -> np.ndarray:
    out = np.zeros((x.shape[0], dp), dtype=np.float32)
    out[:, :x.shape[1]] = x
    return out


def reference_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, dtype: str, layout: str = "HND",
                      causal: bool = False, sm_scale: Optional[float] = None, gran: str = "per_thread",
                      v_dtype: str = "fp8", smooth_k: bool = True, smooth_v: bool = False,
                      cu_seqlens_q: Optional[np.ndarray] = None, cu_seqlens_k: Optional[np.ndarray] = None,
                      rows: Optional[Callable[[int, int], np.ndarray]] = None, want_scores: bool = False,
                      attention: bool = True, bk: int = DEFAULT_BK, exp_band=(0.0, 0.0),
                      want_p: bool = False) -> dict:
    """Run every step of the quantized forward on the CPU.

    q, k, v: float32 arrays holding exact fp16/bf16 values, in the caller's
    layout (HND (B,H,N,D), NHD (B,N,H,D), or packed (T,H,D) with cu_seqlens).
    rows(b, n_b) -> query rows to compute for sequence b (all rows if None).

    Returns a dict with, per sequence b (lists indexed by b):
      q8[b] (Hq, Nq_b, Dp) int8, q_scale[b] (Hq, ceil(Nq_b/Gq)),
      k8[b] (Hkv, Nk_b, Dp), k_scale[b] (Hkv, ceil(Nk_b/Gk)), k_mean[b] (Hkv, Dp),
      v8[b] (Hkv, Nk_b, Dp) uint8 codes (FP8) or v16[b] (Hkv, Nk_b, Dp) float32,
      v_scale[b] (Hkv, Dp), v_mean[b] (Hkv, Dp),
      rows[b], out[b] (Hq, nrows, d) float64, lse[b] (Hq, nrows), scores[b]
      (Hq, nrows, Nk_b) int32 if want_scores, allow[b] (Hq, nrows, d): the most
      that P operands formed from exponents within exp_band = (band_f, band_x)
      of this evaluation's could move each output (see oracle_attn_rows;
      zero for the default band), lse_pq[b] (Hq, nrows): the share of lse due
      to rounding P to its operand format, lse_allow[b] (Hq, nrows): the most
      those operand changes could move lse; with want_p, p[b] (Hq, nrows, Nk_b)
      the P operand of every key at its tile's reference maximum and mref[b]
      (Hq, nrows, Nk_b) float32 that maximum.
    """
    varlen = cu_seqlens_q is not None
    if varlen and cu_seqlens_k is None:
        raise ValueError("varlen needs both cu_seqlens")
    d = q.shape[-1]
    dp = padded_head_dim(d)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    sm32 = float(np.float32(sm_scale))
    gq, gk = Q_GROUP[gran], K_GROUP[gran]
    qp = list(_problems(q, layout, cu_seqlens_q))
    kp = list(_problems(k, layout, cu_seqlens_k))
    vp = list(_problems(v, layout, cu_seqlens_k))
    hq, hkv = qp[0][1].shape[0], kp[0][1].shape[0]
    if hq % hkv:
        raise ValueError("Hq must be divisible by Hkv")
    grp = hq // hkv
    res = {k_: [] for k_ in ("q8", "q_scale", "k8", "k_scale", "k_mean", "v8", "v16", "v_scale", "v_mean",
                             "rows", "out", "lse", "scores", "allow", "lse_pq", "p", "mref", "lse_allow")}
    band_f, band_x = (float(exp_band[0]), float(exp_band[1]))
    L = lib()
    for (b, qb), (_, kb), (_, vb) in zip(qp, kp, vp):
        nq, nk = qb.shape[1], kb.shape[1]
        # K mean, smoothing and INT8 quantization
        k8s, kss, kms = [], [], []
        for h in range(hkv):
            kx = _pad(kb[h], dp)
            km = exact_mean(kx) if smooth_k else np.zeros(dp, dtype=np.float32)
            if smooth_k:
                kx = (kx - km[None, :]).astype(np.float32)
            c, s = quant_int8(kx, nk, gk)
            k8s.append(c); kss.append(s); kms.append(km)
        q8s, qss = [], []
        for h in range(hq):
            c, s = quant_int8(_pad(qb[h], dp), nq, gq)
            q8s.append(c); qss.append(s)
        # V statistics and quantization
        v8s, v16s, vss, vms, vvals = [], [], [], [], []
        for h in range(hkv):
            vx = _pad(vb[h], dp)
            vm = exact_mean(vx) if smooth_v else np.zeros(dp, dtype=np.float32)
            if smooth_v:
                vx = (vx - vm[None, :]).astype(np.float32)
            if v_dtype == "fp8":
                codes, sc = quant_v_fp8(vx)
                v8s.append(codes); vss.append(sc)
                vvals.append(e4m3_decode(codes))
            else:
                vv = vx if not smooth_v else round_half(vx, dtype)
                v16s.append(vv); vvals.append(vv)
            vms.append(vm)
        res["q8"].append(np.stack(q8s)); res["q_scale"].append(np.stack(qss))
        res["k8"].append(np.stack(k8s)); res["k_scale"].append(np.stack(kss)); res["k_mean"].append(np.stack(kms))
        if v_dtype == "fp8":
            res["v8"].append(np.stack(v8s)); res["v_scale"].append(np.stack(vss))
        else:
            res["v16"].append(np.stack(v16s))
        res["v_mean"].append(np.stack(vms))
        if not attention:
            continue
        r = np.arange(nq, dtype=np.int32) if rows is None else np.ascontiguousarray(rows(b, nq), dtype=np.int32)
        res["rows"].append(r)
        outs, lses, scs, alws, lpqs, pds, mds, las = [], [], [], [], [], [], [], []
        p_mode = 0 if v_dtype == "fp8" else (2 if dtype == "bf16" else 1)
        for h in range(hq):
            hk = h // grp
            qs_row = np.ascontiguousarray(np.repeat(qss[h], gq)[:nq], dtype=np.float32)
            ks_key = np.ascontiguousarray(np.repeat(kss[hk], gk)[:nk], dtype=np.float32)
            o = np.zeros((len(r), dp), dtype=np.float64)
            ls = np.zeros(len(r), dtype=np.float64)
            sd = np.zeros((len(r), nk), dtype=np.int32) if want_scores else None
            al = np.zeros((len(r), dp), dtype=np.float64)
            lpq = np.zeros(len(r), dtype=np.float64)
            la = np.zeros(len(r), dtype=np.float64)
            pd = np.zeros((len(r), nk), dtype=np.float64) if want_p else None
            md = np.zeros((len(r), nk), dtype=np.float32) if want_p else None
            vsc = vss[hk] if v_dtype == "fp8" else None
            rc = L.oracle_attn_rows(nq, nk, dp, _p(q8s[h]), _p(qs_row), _p(k8s[hk]), _p(ks_key),
                                    _p(np.ascontiguousarray(vvals[hk], dtype=np.float32)), _p(vsc),
                                    _p(vms[hk] if smooth_v else None), _p(kms[hk] if smooth_k else None),
                                    sm32, int(causal), 0, bk, p_mode, band_f, band_x, len(r), _p(r), _p(o), _p(ls),
                                    _p(sd), _p(al), _p(lpq), _p(pd), _p(md), _p(la))
            if rc != 0:
                raise RuntimeError(f"oracle_attn_rows failed ({rc})")
            outs.append(o[:, :d]); lses.append(ls); alws.append(al[:, :d]); lpqs.append(lpq); las.append(la)
            if want_scores:
                scs.append(sd)
            if want_p:
                pds.append(pd); mds.append(md)
        res["out"].append(np.stack(outs)); res["lse"].append(np.stack(lses)); res["allow"].append(np.stack(alws))
        res["lse_pq"].append(np.stack(lpqs)); res["lse_allow"].append(np.stack(las))
        if want_scores:
            res["scores"].append(np.stack(scs))
        if want_p:
            res["p"].append(np.stack(pds)); res["mref"].append(np.stack(mds))
    return res


def exact_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, layout: str = "HND", causal: bool = False,
                  sm_scale: Optional[float] = None, cu_seqlens_q=None, cu_seqlens_k=None,
                  rows: Optional[Callable[[int, int], np.ndarray]] = None) -> dict:
    """Unquantized attention in fp64 (softmax(QK^T sm_scale) V), same slicing
    and causal convention as reference_forward.  Returns out[b] (Hq, nrows, d)
    and lse[b] (Hq, nrows), natural log."""
    d = q.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    qp = list(_problems(q, layout, cu_seqlens_q))
    kp = list(_problems(k, layout, cu_seqlens_k))
    vp = list(_problems(v, layout, cu_seqlens_k))
    hq, hkv = qp[0][1].shape[0], kp[0][1].shape[0]
    grp = hq // hkv
    res = {"out": [], "lse": [], "rows": []}
    L = lib()
    for (b, qb), (_, kb), (_, vb) in zip(qp, kp, vp):
        nq, nk = qb.shape[1], kb.shape[1]
        r = np.arange(nq, dtype=np.int32) if rows is None else np.ascontiguousarray(rows(b, nq), dtype=np.int32)
        res["rows"].append(r)
        outs, lses = [], []
        for h in range(hq):
            hk = h // grp
            qd = np.ascontiguousarray(qb[h], dtype=np.float64)
            kd = np.ascontiguousarray(kb[hk], dtype=np.float64)
            vd = np.ascontiguousarray(vb[hk], dtype=np.float64)
            o = np.zeros((len(r), d), dtype=np.float64)
            ls = np.zeros(len(r), dtype=np.float64)
            rc = L.oracle_attn_exact(nq, nk, d, _p(qd), _p(kd), _p(vd), float(sm_scale), int(causal), 0,
                                     len(r), _p(r), _p(o), _p(ls))
            if rc != 0:
                raise RuntimeError(f"oracle_attn_exact failed ({rc})")
            outs.append(o); lses.append(ls)
        res["out"].append(np.stack(outs)); res["lse"].append(np.stack(lses))
    return res


def merge_states(out_parts: np.ndarray, lse_parts: np.ndarray):
    """Attention over the union of S disjoint key sets from the S partial
    results (the use of return_lse in [guide] sec. 4.1, Ring-Attention-style
    merging): with o_s the normalised output of set s and L_s its natural-log
    log-sum-exp, exp(L_s) is set s's softmax denominator, so
        out = sum_s exp(L_s - L) o_s,   L = log sum_s exp(L_s).
    Written out in fp64 with the largest L_s as reference point; parts with
    L_s = -inf (no key) weigh 0, and a row with no key at all gives out = 0,
    L = -inf.

    out_parts: (S, R, d) values (decoded fp16/bf16); lse_parts: (S, R).
    Returns out (R, d) and L (R,), fp64."""
    o = np.asarray(out_parts, dtype=np.float64)
    ls = np.asarray(lse_parts, dtype=np.float64)
    m = ls.max(axis=0)
    empty = m == -np.inf
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(ls - m_safe[None, :])                  # exp(-inf) = 0 for empty parts
    W = w.sum(axis=0)
    W_safe = np.where(empty, 1.0, W)
    out = np.einsum("sr,srd->rd", w / W_safe[None, :], o)
    out[empty] = 0.0
    L = np.where(empty, -np.inf, m_safe + np.log(W_safe))
    return out, L


def splitkv_ranges(nk: int, n_splits: int):
    """Key ranges of the split-KV forward as the library defines them: ranges
    of round_up(ceil(nk / n_splits), 128) keys, the last one shorter, none
    empty."""
    per = -(-nk // n_splits)
    slen = -(-per // 128) * 128
    return [(a, min(nk, a + slen)) for a in range(0, nk, slen)]


def reference_forward_splitkv(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, dtype: str, n_splits: int,
                              layout: str = "HND", sm_scale: Optional[float] = None, gran: str = "per_thread",
                              smooth_k: bool = True, smooth_v: bool = False, v_dtype: str = "fp8",
                              rows: Optional[Callable[[int, int], np.ndarray]] = None, exp_band=(0.0, 0.0)) -> dict:
    """The split-KV forward (few queries against many keys; non-causal)
    step by step: quantize Q, K, V over the whole sequence as
    reference_forward does; for each key range (splitkv_ranges) run the
    online-softmax attention of that range alone, starting afresh at its first
    key ([guide] sec. 4.1: q and k/v lengths may differ), keeping its
    normalised output unrounded; combine the ranges with merge_states (the
    return_lse merge of [guide] sec. 4.1).

    Returns per sequence b: out[b] (Hq, nrows, d) fp64 merged output before
    its final rounding, lse[b] (Hq, nrows), allow[b] (Hq, nrows, d): the
    per-range rounding allowances, weighted as in the merge, plus what the
    ranges' LSE allowances
    can move the merge weights (a change of at most e of every L_s moves the
    normalised weights by factors within e^(+-2e)); lse_allow[b]
    (Hq, nrows): the largest LSE allowance of the row's ranges (the merged
    log-sum-exp moves by at most the largest change of its terms);
    parts_scale[b] (Hq, nrows): the largest |range output| of the row;
    rows[b]."""
    d = q.shape[-1]
    dp = padded_head_dim(d)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    sm32 = float(np.float32(sm_scale))
    gq, gk = Q_GROUP[gran], K_GROUP[gran]
    qz = reference_forward(q, k, v, dtype=dtype, layout=layout, gran=gran, v_dtype=v_dtype, smooth_k=smooth_k,
                           smooth_v=smooth_v, attention=False)
    p_mode = 0 if v_dtype == "fp8" else (2 if dtype == "bf16" else 1)
    L = lib()
    res = {"out": [], "lse": [], "allow": [], "lse_allow": [], "parts_scale": [], "rows": []}
    for b in range(len(qz["q8"])):
        q8, qs = qz["q8"][b], qz["q_scale"][b]
        k8, ks, km = qz["k8"][b], qz["k_scale"][b], qz["k_mean"][b]
        vm = qz["v_mean"][b]
        if v_dtype == "fp8":
            v8, vs = qz["v8"][b], qz["v_scale"][b]
        hq, nq = q8.shape[0], q8.shape[1]
        hkv, nk = k8.shape[0], k8.shape[1]
        grp = hq // hkv
        r = np.arange(nq, dtype=np.int32) if rows is None else np.ascontiguousarray(rows(b, nq), dtype=np.int32)
        res["rows"].append(r)
        outs, lses, alws, scs, las = [], [], [], [], []
        for h in range(hq):
            hk = h // grp
            qs_row = np.ascontiguousarray(np.repeat(qs[h], gq)[:nq], dtype=np.float32)
            ks_key = np.repeat(ks[hk], gk)[:nk]
            vval = e4m3_decode(v8[hk]) if v_dtype == "fp8" else qz["v16"][b][hk]
            po, pl, pa, pla = [], [], [], []
            for a0, a1 in splitkv_ranges(nk, n_splits):
                o = np.zeros((len(r), dp), dtype=np.float64)
                ls = np.zeros(len(r), dtype=np.float64)
                al = np.zeros((len(r), dp), dtype=np.float64)
                la = np.zeros(len(r), dtype=np.float64)
                rc = L.oracle_attn_rows(nq, a1 - a0, dp, _p(q8[h]), _p(qs_row),
                                        _p(np.ascontiguousarray(k8[hk][a0:a1])),
                                        _p(np.ascontiguousarray(ks_key[a0:a1], dtype=np.float32)),
                                        _p(np.ascontiguousarray(vval[a0:a1], dtype=np.float32)),
                                        _p(vs[hk] if v_dtype == "fp8" else None),
                                        _p(vm[hk] if smooth_v else None), _p(km[hk] if smooth_k else None),
                                        sm32, 0, 0, DEFAULT_BK, p_mode, float(exp_band[0]), float(exp_band[1]),
                                        len(r), _p(r), _p(o), _p(ls), None, _p(al), None, None, None, _p(la))
                if rc != 0:
                    raise RuntimeError(f"oracle_attn_rows failed ({rc})")
                po.append(o[:, :d])
                pl.append(ls)
                pla.append(la)
                pa.append(al[:, :d])
            po, pl, pa, pla = np.stack(po), np.stack(pl), np.stack(pa), np.stack(pla)
            mo, ml = merge_states(po, pl)
            m = pl.max(axis=0)
            w = np.exp(pl - np.where(np.isneginf(m), 0.0, m)[None, :])
            w = w / np.maximum(w.sum(axis=0), 1e-300)[None, :]
            eps = pla.max(axis=0)
            spread = np.einsum("sr,srd->rd", w, np.abs(po - mo[None]))
            outs.append(mo); lses.append(ml); las.append(eps)
            alws.append(np.einsum("sr,srd->rd", w, pa) + np.expm1(2.0 * eps)[:, None] * spread)
            scs.append(np.abs(po).max(axis=(0, 2)))
        res["out"].append(np.stack(outs)); res["lse"].append(np.stack(lses))
        res["allow"].append(np.stack(alws)); res["parts_scale"].append(np.stack(scs))
        res["lse_allow"].append(np.stack(las))
    return res
