"""Shared helpers for the GPU parity tests: run the HIP path and the CPU
oracle on the same seeded inputs and compare them.

Tolerance for outputs: the GPU's fp16/bf16 output against the oracle's
unrounded value, |diff| <= 2e-3 + one output ulp at |ref| (an fp16/bf16
rounding flip alone can exceed 2e-3 near |ref| ~ 1) + the oracle's rounding
allowance for the exponent band EXP_BAND, plus cosine similarity >= 0.9999;
against exact fp64 attention, cosine similarity >= 0.999.

EXP_BAND.  The kernel forms the exponent of P with a different rounding order
than the oracle: it reads the integer score accumulator, which starts from a
bias B < 2^24, directly as a float (B + S, exactly) and evaluates
x = fl32((B + S) f + fl32(nb - B f)), nb = fl32(log2 448) - m', followed by
v_exp_f32 (1 ulp).  The oracle evaluates x = fl32(s - m'),
s = fl32(fl32(S kscale) c_i), then fl32(2^x) and fl32(. * 448).  Summing the
roundings of both (each |e| <= 2^-24 |value|, the rounding of nb - B f at
most 2^-24 (|nb| + 2^24 f) <= 2^-24 |nb| + f, the maxima of the two score
forms at most 2^-22 |m'| apart, and the exp2 errors), the two values of P
before its operand rounding differ by a factor within 2^(+-delta) with
    delta = f + 2^-21 (|s| + |m'| + 8),   f = c_i kscale_j,
one integer score unit in log2 units plus a relative term.  The oracle's
allowance bounds how far operands formed anywhere in that band can move each
output (it is zero for elements whose P operands cannot change).

LSE: within 1e-3 + the oracle's LSE allowance (what P operands formed within
the exponent band can move ln l: -ln(1 - sum |dP| / l), which matters on rows
with few keys) of the oracle's; against exact fp64 attention within
max_j |s_hat_ij - s_ij| + 1e-3 + that allowance, where s_hat are the
dequantized (unsmoothed) scores and s the exact ones -- log-sum-exp moves by
at most the largest change of its arguments.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

import oracle
import workloads
import quantized_attention_smooth_amd as sage

ABS_TOL = 2e-3
EXP_BAND = (1.0, 2.0 ** -21)
COS_EMU = 0.9999
COS_EXACT = 0.999
LSE_TOL_EMU = 1e-3


def bf16_sum_exact_in_fp64(col: np.ndarray) -> bool:
    """Whether fp64 sums bf16 values exactly in any order: every value is a
    multiple of u, the smallest bf16 ulp among the nonzero values
    (2^(floor(log2|x|) - 7), subnormals 2^-133), so is every partial sum, and
    fp64 holds every multiple of u below 2^53 u; all partial sums are at most
    sum |x|.  The library's bf16 means are bit-exact under this condition."""
    x = np.abs(np.asarray(col, dtype=np.float64))
    nz = x[x != 0]
    if nz.size == 0:
        return True
    u = np.exp2(np.maximum(np.floor(np.log2(nz)), -126.0) - 7.0).min()
    return float(x.sum()) < 2.0 ** 53 * u


def out_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    mbits, emin = (7, -126) if dtype == "bf16" else (10, -14)
    a = np.maximum(np.abs(ref), 2.0 ** emin)
    e = np.floor(np.log2(a))
    return np.exp2(np.maximum(e, emin) - mbits)


def assert_same(actual: np.ndarray, desired: np.ndarray, what: str, inputs: Optional[np.ndarray] = None):
    """Bit-exact comparison that names the first mismatching elements."""
    actual, desired = np.asarray(actual), np.asarray(desired)
    assert actual.shape == desired.shape, (what, actual.shape, desired.shape)
    same = (actual == desired) | (np.isnan(actual) & np.isnan(desired)) if actual.dtype.kind == "f" \
        else (actual == desired)
    if same.all():
        return
    idx = np.argwhere(~same)
    lines = [f"{what}: {len(idx)} of {actual.size} elements differ"]
    for ix in idx[:12]:
        t = tuple(int(i) for i in ix)
        extra = "" if inputs is None else f" input {inputs[t]!r}"
        lines.append(f"  at {t}: gpu {actual[t]!r} oracle {desired[t]!r}{extra}")
    raise AssertionError("\n".join(lines))


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    return float(np.dot(a, b) / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def v_unpermute(vt: np.ndarray, n: int) -> np.ndarray:
    """vt[..., Dp, Nk_pad] in the kernel's key order -> [..., n, Dp].
    Inside each aligned block of 64 keys, key 32b + 8r + 4h + e sits at
    position 32h + 16b + 4r + e (the layout stated in include/sage.h)."""
    k = np.arange(n)
    kk = k & 63
    b, r, h, e = kk >> 5, (kk >> 3) & 3, (kk >> 2) & 1, kk & 3
    pos = (k & ~63) | (h << 5) | (b << 4) | (r << 2) | e
    return np.swapaxes(vt[..., pos], -1, -2)


def written_quant_outputs(qk, qv, lens=None) -> dict:
    """The quantize outputs as a dict of tensors, with, for each varlen
    sequence (lens given), the 128-row tiles after its last one -- which the
    quantizer leaves unwritten -- set to zero, so that two calls' outputs can
    be compared whole."""
    out = {}
    for obj, names in ((qk, ("q8", "q_scale", "k8", "k_scale", "k_mean")), (qv, ("vt", "v_scale", "v_mean"))):
        for f in names:
            x = getattr(obj, f)
            if x is None:
                out[f] = None
                continue
            x = x.clone()
            if lens is not None and f in ("q8", "k8", "q_scale", "k_scale", "vt"):
                axis = 3 if f == "vt" else 2
                rows = x.shape[axis] if f in ("q8", "k8", "vt") else None
                for b, n in enumerate(lens):
                    end = -(-int(n) // 128) * 128
                    if f in ("q_scale", "k_scale"):
                        npad = (qk.q8 if f == "q_scale" else qk.k8).shape[2]
                        end = end * x.shape[axis] // npad
                    elif end > rows:
                        end = rows
                    x[b].narrow(axis - 1, end, x.shape[axis] - end).zero_()
            out[f] = x
    return out


def sample_rows(seed: int, per: int):
    """rows(b, n): the first and last rows, rows around 64/128-row tile edges,
    and a seeded random sample."""
    def f(b, n):
        rng = np.random.default_rng(seed * 1000 + b)
        fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, n // 2, n - 2, n - 1]
        rnd = rng.integers(0, n, size=per)
        r = np.unique(np.clip(np.concatenate([fixed, rnd]), 0, n - 1))
        return r.astype(np.int32)
    return f


class Case:
    """One workload evaluated on both sides."""

    def __init__(self, w: workloads.Workload, inputs: dict, *, v_dtype: Optional[str] = None):
        self.w = w
        self.inp = inputs
        self.v_dtype = v_dtype or w.v_dtype
        self.cu = inputs.get("cu_seqlens")
        self.cu_np = None if self.cu is None else self.cu.numpy()

    # ---------------------------------------------------------------- GPU side
    def run_gpu(self, return_lse: bool = False, sm_scale=None):
        w, dev = self.w, "cuda"
        q, k, v = (self.inp[x].to(dev) for x in ("q", "k", "v"))
        if w.varlen:
            cu = self.cu.to(dev)
            ms = self.inp["max_seqlen"]
            qk = sage.sage_quant_qk(q, k, qk_quant_gran=w.gran, smooth_k=w.smooth_k, cu_seqlens_q=cu,
                                    cu_seqlens_k=cu, max_seqlen_q=ms, max_seqlen_k=ms)
            qv = sage.sage_quant_v(v, v_dtype=self.v_dtype, smooth_v=w.smooth_v, cu_seqlens_k=cu, max_seqlen_k=ms)
            res = sage.sage_attn_varlen_fwd(qk, qv, cu, cu, q.shape[0], is_causal=w.causal, sm_scale=sm_scale,
                                            return_lse=return_lse, pv_accum_dtype=w.pv_accum)
        else:
            qk = sage.sage_quant_qk(q, k, tensor_layout=w.layout, qk_quant_gran=w.gran, smooth_k=w.smooth_k)
            qv = sage.sage_quant_v(v, tensor_layout=w.layout, v_dtype=self.v_dtype, smooth_v=w.smooth_v)
            res = sage.sage_attn_fwd(qk, qv, tensor_layout=w.layout, is_causal=w.causal, sm_scale=sm_scale,
                                     return_lse=return_lse, pv_accum_dtype=w.pv_accum)
        out, lse = (res if return_lse else (res, None))
        torch.cuda.synchronize()
        self.qk, self.qv = qk, qv
        self.gpu_out = out.float().cpu().numpy()
        self.gpu_lse = None if lse is None else lse.cpu().numpy()
        return self

    # ------------------------------------------------------------- oracle side
    def run_oracle(self, rows=None, attention: bool = True, sm_scale=None, exact: bool = False):
        w = self.w
        q, k, v = (self.inp[x].float().numpy() for x in ("q", "k", "v"))
        kw = dict(layout=w.layout, causal=w.causal, sm_scale=sm_scale, cu_seqlens_q=self.cu_np,
                  cu_seqlens_k=self.cu_np, rows=rows)
        self.ref = oracle.reference_forward(q, k, v, dtype=w.dtype, gran=w.gran, v_dtype=self.v_dtype,
                                            smooth_k=w.smooth_k, smooth_v=w.smooth_v, attention=attention,
                                            exp_band=EXP_BAND, **kw)
        self.exact = oracle.exact_forward(q, k, v, **kw) if exact else None
        return self

    # ------------------------------------------------------------- comparisons
    def gpu_rows(self, b: int, rows: np.ndarray) -> np.ndarray:
        """GPU output [Hq, nrows, d] of sequence b at the given rows."""
        o = self.gpu_out
        if self.w.varlen:
            return o[self.cu_np[b] + rows].transpose(1, 0, 2)
        if self.w.layout == "HND":
            return o[b][:, rows]
        return o[b][rows].transpose(1, 0, 2)

    def gpu_lse_rows(self, b: int, rows: np.ndarray) -> np.ndarray:
        if self.w.varlen:
            return self.gpu_lse[:, self.cu_np[b] + rows]
        return self.gpu_lse[b][:, rows]

    def n_seq(self):
        return len(self.ref["q8"])

    def _v_input(self, b: int, nk: int) -> np.ndarray:
        """V of sequence b as (Hkv, nk, d) float32, for error reports."""
        v = self.inp["v"].float().numpy()
        if self.w.varlen:
            return v[self.cu_np[b]:self.cu_np[b] + nk].transpose(1, 0, 2)
        return v[b] if self.w.layout == "HND" else v[b].transpose(1, 0, 2)

    def check_quantized_bitexact(self):
        w = self.w
        gq, gk = oracle.Q_GROUP[w.gran], oracle.K_GROUP[w.gran]
        q8 = self.qk.q8.cpu().numpy()
        qs = self.qk.q_scale.cpu().numpy()
        k8 = self.qk.k8.cpu().numpy()
        ks = self.qk.k_scale.cpu().numpy()
        km = None if self.qk.k_mean is None else self.qk.k_mean.cpu().numpy()
        vt = self.qv.vt.cpu()
        vt = (vt.numpy() if self.v_dtype == "fp8" else vt.float().numpy())
        vs = None if self.qv.v_scale is None else self.qv.v_scale.cpu().numpy()
        vm = None if self.qv.v_mean is None else self.qv.v_mean.cpu().numpy()
        # padding rows are zero up to the end of the sequence's last 128-row
        # tile; for varlen calls the tiles after it are left unwritten
        tile_end = (lambda n, total: -(-n // 128) * 128) if w.varlen else (lambda n, total: total)
        for b in range(self.n_seq()):
            nq = self.ref["q8"][b].shape[1]
            nk = self.ref["k8"][b].shape[1]
            eq, ek = tile_end(nq, q8.shape[2]), tile_end(nk, k8.shape[2])
            np.testing.assert_array_equal(q8[b][:, :nq], self.ref["q8"][b], err_msg=f"q8 seq {b}")
            assert not q8[b][:, nq:eq].any(), "padding rows of q8 must be zero"
            ngq = -(-nq // gq)
            np.testing.assert_array_equal(qs[b][:, :ngq], self.ref["q_scale"][b], err_msg=f"q_scale seq {b}")
            np.testing.assert_array_equal(k8[b][:, :nk], self.ref["k8"][b], err_msg=f"k8 seq {b}")
            assert not k8[b][:, nk:ek].any()
            ngk = -(-nk // gk)
            np.testing.assert_array_equal(ks[b][:, :ngk], self.ref["k_scale"][b], err_msg=f"k_scale seq {b}")
            if w.smooth_k:
                np.testing.assert_array_equal(km[b], self.ref["k_mean"][b], err_msg=f"k_mean seq {b}")
            vb = v_unpermute(vt[b], vt.shape[-1])
            if self.v_dtype == "fp8":
                vin = self._v_input(b, nk)
                assert_same(vb[:, :nk], self.ref["v8"][b], f"v8 seq {b}", vin)
                np.testing.assert_array_equal(vs[b], self.ref["v_scale"][b], err_msg=f"v_scale seq {b}")
            else:
                np.testing.assert_array_equal(vb[:, :nk], self.ref["v16"][b], err_msg=f"v16 seq {b}")
            assert not vb[:, nk:ek].any(), "padding keys of V must be zero"
            if w.smooth_v:
                np.testing.assert_array_equal(vm[b], self.ref["v_mean"][b], err_msg=f"v_mean seq {b}")

    def _problem(self, name: str, b: int) -> np.ndarray:
        """Input tensor of sequence b as (H, n, d) float64."""
        x = self.inp[name].float().numpy()
        if self.w.varlen:
            return x[self.cu_np[b]:self.cu_np[b + 1]].transpose(1, 0, 2).astype(np.float64)
        x = x[b] if self.w.layout == "HND" else x[b].transpose(1, 0, 2)
        return x.astype(np.float64)

    def lse_exact_bound(self, b: int, rows: np.ndarray, sm_scale: float) -> np.ndarray:
        """max_j |s_hat_ij - s_ij| per (head, row): dequantized unsmoothed
        scores against exact ones (natural-log units)."""
        gq, gk = oracle.Q_GROUP[self.w.gran], oracle.K_GROUP[self.w.gran]
        q, k = self._problem("q", b), self._problem("k", b)
        d = q.shape[-1]
        grp = q.shape[0] // k.shape[0]
        out = np.zeros((q.shape[0], len(rows)))
        for h in range(q.shape[0]):
            hk = h // grp
            qs = np.repeat(self.ref["q_scale"][b][h], gq)[rows].astype(np.float64)
            qh = self.ref["q8"][b][h][rows, :d].astype(np.float64) * qs[:, None]
            nk = k.shape[1]
            ks = np.repeat(self.ref["k_scale"][b][hk], gk)[:nk].astype(np.float64)
            kh = self.ref["k8"][b][hk][:, :d].astype(np.float64) * ks[:, None]
            kh = kh + self.ref["k_mean"][b][hk][None, :d].astype(np.float64)
            s_hat = qh @ kh.T * sm_scale
            s = q[h][rows] @ k[hk].T * sm_scale
            out[h] = np.abs(s_hat - s).max(axis=1)
        return out

    def check_outputs(self, lse: bool = False, sm_scale=None):
        worst = 0.0
        gs, rs, es = [], [], []
        sm = sm_scale if sm_scale is not None else 1.0 / math.sqrt(self.w.d)
        for b in range(self.n_seq()):
            rows = self.ref["rows"][b]
            g = self.gpu_rows(b, rows)
            r = self.ref["out"][b]
            tol = ABS_TOL + out_ulp(r, self.w.dtype) + self.ref["allow"][b]
            err = np.abs(g - r)
            bad = err > tol
            assert not bad.any(), (f"seq {b}: {bad.sum()} outputs out of tolerance, max err "
                                   f"{err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}")
            worst = max(worst, float((err - ABS_TOL).max()))
            gs.append(g.ravel()); rs.append(r.ravel())
            if self.exact is not None:
                es.append(self.exact["out"][b].ravel())
            if lse:
                gl = self.gpu_lse_rows(b, rows)
                lerr = np.abs(gl - self.ref["lse"][b])
                ltol = LSE_TOL_EMU + self.ref["lse_allow"][b]
                assert np.all(lerr <= ltol), (f"seq {b}: lse off by {lerr.max():.3g} at "
                                              f"{np.unravel_index(lerr.argmax(), lerr.shape)}")
                if self.exact is not None and self.w.smooth_k:
                    # score error of the INT8 Q/K, plus what rounding P to its
                    # operand format moved the row sum, plus the emulation slack
                    bound = (self.lse_exact_bound(b, rows, sm) + self.ref["lse_pq"][b] + LSE_TOL_EMU + 1e-4 +
                             self.ref["lse_allow"][b])
                    assert np.all(np.abs(gl - self.exact["lse"][b]) <= bound)
        g, r = np.concatenate(gs), np.concatenate(rs)
        c_emu = cosine(g, r)
        assert c_emu >= COS_EMU, c_emu
        c_ex = None
        if es:
            c_ex = cosine(g, np.concatenate(es))
            assert c_ex >= COS_EXACT, c_ex
        return c_emu, c_ex


def scale_down(name: str, **kw) -> dict:
    return workloads.make_inputs(workloads.WORKLOADS[name], scale_down=kw or None)
