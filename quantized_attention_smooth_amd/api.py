"""Python binding of the C ABI (include/sage.h).

torch is used only to allocate device memory and to take the current HIP
stream; every computation runs in libsage.so's gfx950 kernels.  The entry
points carry the C names (sage_quant_qk, sage_quant_v, sage_attn_fwd,
sage_attn_varlen_fwd); sageattn / sageattn_varlen chain them the way the
SageAttention deployment guide's API is used (pwwt.cn, sec. 4.1 signature:
q, k, v, tensor_layout, is_causal, sm_scale, return_lse; sec. 4.2 knobs:
qk_quant_gran, pv_accum_dtype, smooth_k, smooth_v; sageattn_varlen with
cu_seqlens_q / cu_seqlens_k).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional

import torch

from . import _abi as A

_GRAN = {"per_block": A.SAGE_PER_BLOCK, "per_warp": A.SAGE_PER_WARP, "per_thread": A.SAGE_PER_THREAD}
_QG = {"per_block": 128, "per_warp": 32, "per_thread": 1}
_KG = {"per_block": 64, "per_warp": 64, "per_thread": 16}
_ACC = {"fp32": A.SAGE_ACC_FP32, "fp16": A.SAGE_ACC_FP16, "fp16+fp32": A.SAGE_ACC_FP16_FP32,
        "fp32+fp16": A.SAGE_ACC_FP16_FP32, "fp32+fp32": A.SAGE_ACC_FP32_FP32}
_DT = {torch.float16: A.SAGE_F16, torch.bfloat16: A.SAGE_BF16}
PAD = 128


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def padded_head_dim(d: int) -> int:
    if d < 1 or d > 128:
        raise ValueError(f"head_dim {d} unsupported: must be 1..128 (deployment guide sec. 4.1)")
    return 64 if d <= 64 else 128


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


@dataclasses.dataclass
class Geometry:
    B: int
    H: int
    N: int
    d: int
    sb: int
    sh: int
    sn: int


def _geometry(x: torch.Tensor, layout: str, cu: Optional[torch.Tensor], max_seqlen: Optional[int]) -> Geometry:
    if x.dtype not in _DT:
        raise ValueError(f"dtype {x.dtype} unsupported: fp16 or bf16")
    if x.stride(-1) != 1:
        raise ValueError("the last (head_dim) dimension must be contiguous")
    if cu is not None:
        if x.dim() != 3:
            raise ValueError("varlen tensors are packed (total_tokens, heads, head_dim)")
        if max_seqlen is None:
            c = cu.to("cpu")
            max_seqlen = int((c[1:] - c[:-1]).max())
        return Geometry(cu.numel() - 1, x.shape[1], int(max_seqlen), x.shape[2], 0, x.stride(1), x.stride(0))
    if x.dim() != 4:
        raise ValueError("dense tensors are 4-D (HND or NHD)")
    if layout == "HND":
        return Geometry(x.shape[0], x.shape[1], x.shape[2], x.shape[3], x.stride(0), x.stride(1), x.stride(2))
    if layout == "NHD":
        return Geometry(x.shape[0], x.shape[2], x.shape[1], x.shape[3], x.stride(0), x.stride(2), x.stride(1))
    raise ValueError(f"tensor_layout must be 'HND' or 'NHD', not {layout!r}")


def _check_out(out: torch.Tensor, shape, device: torch.device, name: str = "out") -> None:
    """A caller-supplied output must have exactly the extent the kernels write
    (the C ABI sees only its pointer and strides), a 16-bit float dtype, the
    inputs' device and a contiguous last dimension."""
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(out.shape)}, expected {tuple(shape)}")
    if out.dtype not in _DT:
        raise ValueError(f"{name} dtype {out.dtype} unsupported: fp16 or bf16")
    if out.device != device:
        raise ValueError(f"{name} is on {out.device}, the inputs on {device}")
    if out.stride(-1) != 1:
        raise ValueError(f"the last dimension of {name} must be contiguous")


@dataclasses.dataclass
class QuantQK:
    """Quantized K with INT8 Q (q8, q_scale) or, for an attention call that
    quantizes Q itself, Q in its input precision (q and its element strides
    (b, h, n); q8 and q_scale None)."""
    q8: Optional[torch.Tensor]
    q_scale: Optional[torch.Tensor]
    k8: torch.Tensor
    k_scale: torch.Tensor
    k_mean: Optional[torch.Tensor]
    gran: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: torch.dtype
    q: Optional[torch.Tensor] = None
    q_strides: tuple = (0, 0, 0)

    @property
    def device(self) -> torch.device:
        return self.k8.device


@dataclasses.dataclass
class QuantV:
    vt: torch.Tensor
    v_scale: Optional[torch.Tensor]
    v_mean: Optional[torch.Tensor]
    v_dtype: str


def workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(A.load().sage_quant_workspace_size(B, H, N, d))


def _quant_qk_params(q: torch.Tensor, k: torch.Tensor, tensor_layout: str, qk_quant_gran: str, smooth_k: bool,
                     cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, workspace, alloc_workspace=True,
                     quantize_q=True):
    if qk_quant_gran not in _GRAN:
        raise ValueError(f"qk_quant_gran must be one of {sorted(_GRAN)}")
    if q.dtype != k.dtype or q.device != k.device:
        raise ValueError("q and k must share dtype and device")
    gq = _geometry(q, tensor_layout, cu_seqlens_q, max_seqlen_q)
    gk = _geometry(k, tensor_layout, cu_seqlens_k, max_seqlen_k)
    if gq.d != gk.d or gq.B != gk.B:
        raise ValueError("q and k must share batch and head_dim")
    dp = padded_head_dim(gq.d)
    dev = q.device
    nq_pad, nk_pad = _round_up(gq.N, PAD), _round_up(gk.N, PAD)
    if quantize_q:
        q8 = torch.empty((gq.B, gq.H, nq_pad, dp), dtype=torch.int8, device=dev)
        qs = torch.empty((gq.B, gq.H, nq_pad // _QG[qk_quant_gran]), dtype=torch.float32, device=dev)
    else:
        q8 = qs = None
    k8 = torch.empty((gk.B, gk.H, nk_pad, dp), dtype=torch.int8, device=dev)
    ks = torch.empty((gk.B, gk.H, nk_pad // _KG[qk_quant_gran]), dtype=torch.float32, device=dev)
    km = torch.empty((gk.B, gk.H, dp), dtype=torch.float32, device=dev) if smooth_k else None
    if smooth_k and workspace is None and alloc_workspace:
        workspace = torch.empty(workspace_bytes(gk.B, gk.H, gk.N, gk.d), dtype=torch.uint8, device=dev)
    p = A.QuantQKParams()
    p.struct_size = ctypes.sizeof(A.QuantQKParams)
    p.q, p.k, p.dtype = _ptr(q) if quantize_q else None, _ptr(k), _DT[q.dtype]
    p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d = gq.B, gq.H, gk.H, gq.N, gk.N, gq.d
    p.q_stride_b, p.q_stride_h, p.q_stride_n = gq.sb, gq.sh, gq.sn
    p.k_stride_b, p.k_stride_h, p.k_stride_n = gk.sb, gk.sh, gk.sn
    p.cu_seqlens_q, p.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    p.gran, p.smooth_k = _GRAN[qk_quant_gran], int(bool(smooth_k))
    p.q8, p.q_scale, p.k8, p.k_scale, p.k_mean = _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks), _ptr(km)
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    res = QuantQK(q8, qs, k8, ks, km, qk_quant_gran, gq.B, gq.H, gk.H, gq.N, gk.N, gq.d, q.dtype,
                  None if quantize_q else q, (gq.sb, gq.sh, gq.sn))
    return p, res, workspace


def _quant_v_params(v: torch.Tensor, tensor_layout: str, v_dtype: str, smooth_v: bool, cu_seqlens_k, max_seqlen_k,
                    workspace, alloc_workspace=True):
    if v_dtype not in ("fp8", "fp16"):
        raise ValueError("v_dtype must be 'fp8' or 'fp16' (the input's 16-bit type)")
    g = _geometry(v, tensor_layout, cu_seqlens_k, max_seqlen_k)
    dp = padded_head_dim(g.d)
    dev = v.device
    nk_pad = _round_up(g.N, PAD)
    fp8 = v_dtype == "fp8"
    vt = torch.empty((g.B, g.H, dp, nk_pad), dtype=torch.uint8 if fp8 else v.dtype, device=dev)
    vs = torch.empty((g.B, g.H, dp), dtype=torch.float32, device=dev) if fp8 else None
    vm = torch.empty((g.B, g.H, dp), dtype=torch.float32, device=dev) if smooth_v else None
    if (fp8 or smooth_v) and workspace is None and alloc_workspace:
        workspace = torch.empty(workspace_bytes(g.B, g.H, g.N, g.d), dtype=torch.uint8, device=dev)
    p = A.QuantVParams()
    p.struct_size = ctypes.sizeof(A.QuantVParams)
    p.v, p.dtype = _ptr(v), _DT[v.dtype]
    p.B, p.Hkv, p.Nk, p.d = g.B, g.H, g.N, g.d
    p.v_stride_b, p.v_stride_h, p.v_stride_n = g.sb, g.sh, g.sn
    p.cu_seqlens_k = _ptr(cu_seqlens_k)
    p.v_dtype = A.SAGE_V_FP8 if fp8 else A.SAGE_V_FP16
    p.smooth_v = int(bool(smooth_v))
    p.vt, p.v_scale, p.v_mean = _ptr(vt), _ptr(vs), _ptr(vm)
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return p, QuantV(vt, vs, vm, v_dtype), workspace


def sage_quant_qk(q: torch.Tensor, k: torch.Tensor, *, tensor_layout: str = "HND",
                  qk_quant_gran: str = "per_thread", smooth_k: bool = True,
                  cu_seqlens_q: Optional[torch.Tensor] = None, cu_seqlens_k: Optional[torch.Tensor] = None,
                  max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                  workspace: Optional[torch.Tensor] = None) -> QuantQK:
    L = A.load()
    p, res, _ = _quant_qk_params(q, k, tensor_layout, qk_quant_gran, smooth_k, cu_seqlens_q, cu_seqlens_k,
                                 max_seqlen_q, max_seqlen_k, workspace)
    A.check(L.sage_quant_qk(ctypes.byref(p), _stream()))
    return res


def sage_quant_v(v: torch.Tensor, *, tensor_layout: str = "HND", v_dtype: str = "fp8", smooth_v: bool = False,
                 cu_seqlens_k: Optional[torch.Tensor] = None, max_seqlen_k: Optional[int] = None,
                 workspace: Optional[torch.Tensor] = None) -> QuantV:
    L = A.load()
    p, res, _ = _quant_v_params(v, tensor_layout, v_dtype, smooth_v, cu_seqlens_k, max_seqlen_k, workspace)
    A.check(L.sage_quant_v(ctypes.byref(p), _stream()))
    return res


def sage_quant_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, tensor_layout: str = "HND",
                   qk_quant_gran: str = "per_thread", smooth_k: bool = True, v_dtype: str = "fp8",
                   smooth_v: bool = False, cu_seqlens_q: Optional[torch.Tensor] = None,
                   cu_seqlens_k: Optional[torch.Tensor] = None, max_seqlen_q: Optional[int] = None,
                   max_seqlen_k: Optional[int] = None, workspace_k: Optional[torch.Tensor] = None,
                   workspace_v: Optional[torch.Tensor] = None, quantize_q: bool = True):
    """sage_quant_qk and sage_quant_v in one call (two kernel launches);
    the K and V workspaces, when given, must be distinct buffers.  With
    quantize_q=False, Q is left in its input precision for an attention call
    that quantizes it itself (see q_fusable)."""
    L = A.load()
    if v.dtype != k.dtype or v.device != k.device:
        raise ValueError("k and v must share dtype and device")
    pk, rqk, _ = _quant_qk_params(q, k, tensor_layout, qk_quant_gran, smooth_k, cu_seqlens_q, cu_seqlens_k,
                                  max_seqlen_q, max_seqlen_k, workspace_k, quantize_q=quantize_q)
    pv, rv, _ = _quant_v_params(v, tensor_layout, v_dtype, smooth_v, cu_seqlens_k, max_seqlen_k, workspace_v)
    A.check(L.sage_quant_qkv(ctypes.byref(pk), ctypes.byref(pv), _stream()))
    return rqk, rv


class QuantQKVPlan:
    """sage_quant_qkv with its outputs, workspaces and parameter blocks made
    once: run() launches the two quantize kernels into the same output tensors
    on the current stream each time, for loops over inputs of one shape held
    in the same buffers (each run overwrites the previous results).  qk and qv
    are the outputs, as sage_quant_qkv returns them."""

    def __init__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, **kw):
        self._keep = (q, k, v, kw.get("cu_seqlens_q"), kw.get("cu_seqlens_k"))
        layout = kw.pop("tensor_layout", "HND")
        gran = kw.pop("qk_quant_gran", "per_thread")
        smooth_k = kw.pop("smooth_k", True)
        v_dtype = kw.pop("v_dtype", "fp8")
        smooth_v = kw.pop("smooth_v", False)
        cq, ck = kw.pop("cu_seqlens_q", None), kw.pop("cu_seqlens_k", None)
        mq, mk = kw.pop("max_seqlen_q", None), kw.pop("max_seqlen_k", None)
        quantize_q = kw.pop("quantize_q", True)
        if kw:
            raise TypeError(f"unexpected arguments {sorted(kw)}")
        if v.dtype != k.dtype or v.device != k.device:
            raise ValueError("k and v must share dtype and device")
        self._pk, self.qk, self._wk = _quant_qk_params(q, k, layout, gran, smooth_k, cq, ck, mq, mk, None,
                                                       quantize_q=quantize_q)
        self._pv, self.qv, self._wv = _quant_v_params(v, layout, v_dtype, smooth_v, ck, mk, None)
        self._L = A.load()

    def run(self):
        A.check(self._L.sage_quant_qkv(ctypes.byref(self._pk), ctypes.byref(self._pv), _stream()))
        return self.qk, self.qv


def sage_quant_qkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, tensor_layout: str = "HND",
                           qk_quant_gran: str = "per_thread", smooth_k: bool = True, v_dtype: str = "fp8",
                           smooth_v: bool = False, cu_seqlens_q: Optional[torch.Tensor] = None,
                           cu_seqlens_k: Optional[torch.Tensor] = None, max_seqlen_q: Optional[int] = None,
                           max_seqlen_k: Optional[int] = None):
    """sage_quant_qkv with the statistics partials in the library's static
    device array instead of a workspace (for callers that cannot allocate;
    calls that overlap on one GPU race on that array).  The outputs are
    allocated here, as for the other calls."""
    L = A.load()
    if v.dtype != k.dtype or v.device != k.device:
        raise ValueError("k and v must share dtype and device")
    pk, rqk, _ = _quant_qk_params(q, k, tensor_layout, qk_quant_gran, smooth_k, cu_seqlens_q, cu_seqlens_k,
                                  max_seqlen_q, max_seqlen_k, None, alloc_workspace=False)
    pv, rv, _ = _quant_v_params(v, tensor_layout, v_dtype, smooth_v, cu_seqlens_k, max_seqlen_k, None,
                                alloc_workspace=False)
    A.check(L.sage_quant_qkv_noalloc(ctypes.byref(pk), ctypes.byref(pv), _stream()))
    return rqk, rv


def _attn_params(qk: QuantQK, qv: QuantV, out: torch.Tensor, lse: Optional[torch.Tensor], is_causal: bool,
                 sm_scale: Optional[float], pv_accum_dtype: str, strides) -> A.AttnParams:
    if pv_accum_dtype not in _ACC:
        raise ValueError(f"pv_accum_dtype must be one of {sorted(_ACC)}")
    p = A.AttnParams()
    p.struct_size = ctypes.sizeof(A.AttnParams)
    p.q8, p.q_scale, p.k8, p.k_scale, p.k_mean = _ptr(qk.q8), _ptr(qk.q_scale), _ptr(qk.k8), _ptr(qk.k_scale), _ptr(qk.k_mean)
    if qk.q is not None:
        p.q = _ptr(qk.q)
        p.q_stride_b, p.q_stride_h, p.q_stride_n = qk.q_strides
    p.vt, p.v_scale, p.v_mean = _ptr(qv.vt), _ptr(qv.v_scale), _ptr(qv.v_mean)
    p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d = qk.B, qk.Hq, qk.Hkv, qk.Nq, qk.Nk, qk.d
    p.gran = _GRAN[qk.gran]
    p.v_dtype = A.SAGE_V_FP8 if qv.v_dtype == "fp8" else A.SAGE_V_FP16
    p.pv_accum = _ACC[pv_accum_dtype]
    p.is_causal = int(bool(is_causal))
    p.sm_scale = float(sm_scale) if sm_scale is not None else 0.0
    p.in_dtype = _DT[qk.dtype]
    p.out, p.out_dtype = _ptr(out), _DT[out.dtype]
    p.o_stride_b, p.o_stride_h, p.o_stride_n = strides
    p.lse = _ptr(lse)
    return p


def sage_attn_fwd(qk: QuantQK, qv: QuantV, *, tensor_layout: str = "HND", is_causal: bool = False,
                  sm_scale: Optional[float] = None, return_lse: bool = False, pv_accum_dtype: str = "fp32+fp32",
                  out: Optional[torch.Tensor] = None):
    L = A.load()
    dev = qk.device
    if tensor_layout not in ("HND", "NHD"):
        raise ValueError(f"tensor_layout must be 'HND' or 'NHD', not {tensor_layout!r}")
    shape = (qk.B, qk.Hq, qk.Nq, qk.d) if tensor_layout == "HND" else (qk.B, qk.Nq, qk.Hq, qk.d)
    if out is None:
        out = torch.empty(shape, dtype=qk.dtype, device=dev)
    else:
        _check_out(out, shape, dev)
    g = _geometry(out, tensor_layout, None, None)
    lse = torch.empty((qk.B, qk.Hq, qk.Nq), dtype=torch.float32, device=dev) if return_lse else None
    p = _attn_params(qk, qv, out, lse, is_causal, sm_scale, pv_accum_dtype, (g.sb, g.sh, g.sn))
    A.check(L.sage_attn_fwd(ctypes.byref(p), _stream()))
    return (out, lse) if return_lse else out


PACK_MAX_NQ = 128       # the library packs the query heads of a K/V head together up to this many queries
MI355X_CUS = 256        # compute units of one MI355X


def splitkv_plan(B: int, Hq: int, Nq: int, Nk: int, n_splits: Optional[int] = None, Hkv: Optional[int] = None,
                 cus: int = MI355X_CUS) -> int:
    """Number of key ranges to ask for: as many as fit one round of
    workgroups, one per compute unit (an attention workgroup takes a whole
    CU), with ranges of at least 256 keys and at most 64 ranges.  A second,
    partial round would leave most CUs idle while it runs.  With grouped K/V
    heads and few queries, the library runs the rows of all query heads of a
    K/V head in one workgroup, so there are fewer row tiles."""
    if n_splits is not None:
        return int(n_splits)
    Hkv = Hq if Hkv is None else Hkv
    if Hq > Hkv and Nq <= PACK_MAX_NQ:
        tiles = B * Hkv * ((Hq // Hkv * Nq + 255) // 256)
    else:
        tiles = B * Hq * ((Nq + 255) // 256)
    return max(1, min(64, cus // tiles, Nk // 256))


def sage_attn_fwd_splitkv(qk: QuantQK, qv: QuantV, *, n_splits: Optional[int] = None, tensor_layout: str = "HND",
                          sm_scale: Optional[float] = None, return_lse: bool = False,
                          pv_accum_dtype: str = "fp32+fp32", out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None):
    """sage_attn_fwd with the keys cut into ranges that run in parallel and are
    merged by their log-sum-exp (few queries, many keys; non-causal)."""
    L = A.load()
    dev = qk.device
    if tensor_layout not in ("HND", "NHD"):
        raise ValueError(f"tensor_layout must be 'HND' or 'NHD', not {tensor_layout!r}")
    shape = (qk.B, qk.Hq, qk.Nq, qk.d) if tensor_layout == "HND" else (qk.B, qk.Nq, qk.Hq, qk.d)
    if out is None:
        out = torch.empty(shape, dtype=qk.dtype, device=dev)
    else:
        _check_out(out, shape, dev)
    g = _geometry(out, tensor_layout, None, None)
    lse = torch.empty((qk.B, qk.Hq, qk.Nq), dtype=torch.float32, device=dev) if return_lse else None
    ns = splitkv_plan(qk.B, qk.Hq, qk.Nq, qk.Nk, n_splits, qk.Hkv)
    need = int(L.sage_attn_splitkv_workspace_size(qk.B, qk.Hq, qk.Nq, qk.Nk, qk.d, ns))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    p = _attn_params(qk, qv, out, lse, False, sm_scale, pv_accum_dtype, (g.sb, g.sh, g.sn))
    A.check(L.sage_attn_fwd_splitkv(ctypes.byref(p), ns, _ptr(workspace), workspace.numel(), _stream()))
    return (out, lse) if return_lse else out


def sage_attn_varlen_fwd(qk: QuantQK, qv: QuantV, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                         total_q: int, *, is_causal: bool = False, sm_scale: Optional[float] = None,
                         return_lse: bool = False, pv_accum_dtype: str = "fp32+fp32",
                         out: Optional[torch.Tensor] = None):
    L = A.load()
    dev = qk.device
    if out is None:
        out = torch.empty((total_q, qk.Hq, qk.d), dtype=qk.dtype, device=dev)
    else:
        _check_out(out, (total_q, qk.Hq, qk.d), dev)
    lse = torch.empty((qk.Hq, total_q), dtype=torch.float32, device=dev) if return_lse else None
    vp = A.AttnVarlenParams()
    vp.base = _attn_params(qk, qv, out, lse, is_causal, sm_scale, pv_accum_dtype, (0, out.stride(1), out.stride(0)))
    vp.base.struct_size = ctypes.sizeof(A.AttnVarlenParams)
    vp.cu_seqlens_q, vp.cu_seqlens_k, vp.total_q = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(total_q)
    A.check(L.sage_attn_varlen_fwd(ctypes.byref(vp), _stream()))
    return (out, lse) if return_lse else out


def sage_debug_qk_scores(qk: QuantQK, checksums: bool = False, cu_seqlens_q: Optional[torch.Tensor] = None,
                         cu_seqlens_k: Optional[torch.Tensor] = None, total_q: Optional[int] = None) -> torch.Tensor:
    """int32 scores [B, Hq, Nq, Nk] from the attention kernel's QK^T tile code,
    or int64 row checksums [B, Hq, Nq, 2] (sum_j S_ij, sum_j (j+1) S_ij).  For
    a varlen batch (cu_seqlens given) only the checksums exist, int64
    [Hq, total_q, 2], over each row's own sequence."""
    L = A.load()
    dev = qk.device
    if qk.q8 is None:
        raise ValueError("the score dump reads the INT8 Q of sage_quant_qk (quantize_q=True)")
    if cu_seqlens_q is not None:
        if not checksums or cu_seqlens_k is None or total_q is None:
            raise ValueError("varlen scores come as checksums, with cu_seqlens_q, cu_seqlens_k and total_q")
        buf = torch.empty((qk.Hq, int(total_q), 2), dtype=torch.int64, device=dev)
        vp = A.AttnVarlenParams()
        vp.base.struct_size = ctypes.sizeof(A.AttnVarlenParams)
        vp.base.q8, vp.base.k8 = _ptr(qk.q8), _ptr(qk.k8)
        vp.base.B, vp.base.Hq, vp.base.Hkv, vp.base.Nq, vp.base.Nk, vp.base.d = qk.B, qk.Hq, qk.Hkv, qk.Nq, qk.Nk, qk.d
        vp.base.gran = _GRAN[qk.gran]
        vp.cu_seqlens_q, vp.cu_seqlens_k, vp.total_q = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(total_q)
        A.check(L.sage_debug_qk_scores_varlen(ctypes.byref(vp), _ptr(buf), _stream()))
        return buf
    if checksums:
        buf = torch.empty((qk.B, qk.Hq, qk.Nq, 2), dtype=torch.int64, device=dev)
    else:
        buf = torch.empty((qk.B, qk.Hq, qk.Nq, qk.Nk), dtype=torch.int32, device=dev)
    p = A.AttnParams()
    p.struct_size = ctypes.sizeof(A.AttnParams)
    p.q8, p.k8 = _ptr(qk.q8), _ptr(qk.k8)
    p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d = qk.B, qk.Hq, qk.Hkv, qk.Nq, qk.Nk, qk.d
    p.gran = _GRAN[qk.gran]
    A.check(L.sage_debug_qk_scores(ctypes.byref(p), 1 if checksums else 0, _ptr(buf), _stream()))
    return buf


def sage_merge_states(out_parts: torch.Tensor, lse_parts: torch.Tensor, *, tensor_layout: str = "HND",
                      return_lse: bool = True, out: Optional[torch.Tensor] = None):
    """Combine attention results over S disjoint key sets of the same queries
    (the consumer of return_lse, deployment guide sec. 4.1).

    out_parts: fp16/bf16 [S, B, H, N, d] (HND) or [S, B, N, H, d] (NHD), the
    normalised outputs of the S sets; lse_parts: fp32 [S, B, H, N], their
    natural-log LSEs.  Returns out (layout of one part) and, with return_lse,
    the merged fp32 LSE [B, H, N]."""
    L = A.load()
    if out_parts.dim() != 5 or lse_parts.dim() != 4:
        raise ValueError("out_parts must be 5-D [S, ...] and lse_parts 4-D [S, B, H, N]")
    if out_parts.dtype not in _DT:
        raise ValueError("out_parts must be fp16 or bf16")
    if lse_parts.dtype != torch.float32 or not lse_parts.is_contiguous():
        raise ValueError("lse_parts must be contiguous fp32")
    if out_parts.stride(-1) != 1:
        raise ValueError("the last dimension of out_parts must be contiguous")
    S = out_parts.shape[0]
    if tensor_layout == "HND":
        _, B, H, N, d = out_parts.shape
        ps = (out_parts.stride(0), out_parts.stride(1), out_parts.stride(2), out_parts.stride(3))
    elif tensor_layout == "NHD":
        _, B, N, H, d = out_parts.shape
        ps = (out_parts.stride(0), out_parts.stride(1), out_parts.stride(3), out_parts.stride(2))
    else:
        raise ValueError(f"tensor_layout must be HND or NHD, got {tensor_layout!r}")
    if tuple(lse_parts.shape) != (S, B, H, N):
        raise ValueError(f"lse_parts shape {tuple(lse_parts.shape)} != {(S, B, H, N)}")
    if out is None:
        out = torch.empty(out_parts.shape[1:], dtype=out_parts.dtype, device=out_parts.device)
    else:
        _check_out(out, out_parts.shape[1:], out_parts.device)
        if out.dtype != out_parts.dtype:
            raise ValueError(f"out dtype {out.dtype} differs from the parts' {out_parts.dtype}")
    os_ = (out.stride(0), out.stride(1), out.stride(2)) if tensor_layout == "HND" else \
        (out.stride(0), out.stride(2), out.stride(1))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=out_parts.device) if return_lse else None
    p = A.MergeParams()
    p.struct_size = ctypes.sizeof(A.MergeParams)
    p.n_parts, p.dtype, p.B, p.H, p.N, p.d = S, _DT[out_parts.dtype], B, H, N, d
    p.parts = _ptr(out_parts)
    p.ps_s, p.ps_b, p.ps_h, p.ps_n = ps
    p.lse_parts = _ptr(lse_parts)
    p.out = _ptr(out)
    p.o_stride_b, p.o_stride_h, p.o_stride_n = os_
    p.lse = _ptr(lse)
    A.check(L.sage_merge_states(ctypes.byref(p), _stream()))
    return (out, lse) if return_lse else out


def q_fusable(q: torch.Tensor, B: int, Hq: int, Hkv: int, Nq: int, d: int, qk_quant_gran: str, v_dtype: str,
              is_causal: bool, varlen: bool, strides) -> bool:
    """Whether the attention call takes this Q in its input precision and
    quantizes it in its own kernel (sage_attn_q_fusable for the sizes, a
    16-byte aligned q, strides in multiples of 8 elements)."""
    if qk_quant_gran not in _GRAN or v_dtype not in ("fp8", "fp16"):
        return False
    L = A.load()
    vd = A.SAGE_V_FP8 if v_dtype == "fp8" else A.SAGE_V_FP16
    if not L.sage_attn_q_fusable(B, Hq, Hkv, Nq, d, _GRAN[qk_quant_gran], vd, int(bool(is_causal)), int(varlen)):
        return False
    sb, sh, sn = strides
    return q.data_ptr() % 16 == 0 and sh % 8 == 0 and sn % 8 == 0 and (varlen or sb % 8 == 0)


AUTO_MIN_KEYS_PER_RANGE = 1024


def auto_kv_splits(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, is_causal: bool, kv_splits="auto") -> int:
    """Number of key ranges sageattn runs: 1 is the one-pass forward.
    "auto" splits a non-causal call whose row tiles leave compute units idle
    (splitkv_plan gives at least 2 ranges: few queries against many keys),
    into ranges of at least AUTO_MIN_KEYS_PER_RANGE keys: shorter ranges
    leave each workgroup too little work beside its fixed costs, and every
    range rounds its own P, so a small call stays one pass.  None or 1 is one
    pass; an int n >= 2 asks for n ranges (non-causal only)."""
    if kv_splits is None:
        return 1
    if kv_splits == "auto":
        if is_causal:
            return 1
        n = min(splitkv_plan(B, Hq, Nq, Nk, None, Hkv), Nk // AUTO_MIN_KEYS_PER_RANGE)
        return n if n >= 2 else 1
    n = int(kv_splits)
    if n < 1:
        raise ValueError("kv_splits must be 'auto', None or an int >= 1")
    if n > 1 and is_causal:
        raise NotImplementedError("kv_splits needs a non-causal call")
    return n


def sageattn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tensor_layout="HND", is_causal=False,
             sm_scale: Optional[float] = None, return_lse=False, *, qk_quant_gran: str = "per_thread",
             pv_accum_dtype: str = "fp32+fp32", smooth_k: bool = True, smooth_v: bool = False, v_dtype: str = "fp8",
             kv_splits="auto", attn_mask=None, dropout_p: float = 0.0, scale: Optional[float] = None,
             enable_gqa: Optional[bool] = None):
    """Quantized attention forward: out = softmax(q k^T * sm_scale) v.

    q, k, v: fp16/bf16 CUDA tensors, (B, H, N, D) for HND or (B, N, H, D) for
    NHD, same dtype; Hq must be a multiple of Hkv; D <= 128.
    kv_splits: "auto" (default) runs the split-KV forward (key ranges in
    parallel, merged by log-sum-exp) when a non-causal call has too few row
    tiles to fill the GPU -- few queries against many keys -- and one pass
    over the keys otherwise; None or 1 always runs one pass; an int n >= 2
    asks for n ranges (non-causal only).
    Returns out (same dtype and layout as q) and, with return_lse, the fp32
    log-sum-exp [B, Hq, Nq].

    Drop-in for torch.nn.functional.scaled_dot_product_attention (deployment
    guide sec. 5.1 assigns sageattn to it): SDPA's keywords attn_mask,
    dropout_p, is_causal, scale and enable_gqa are accepted, and so is SDPA's
    positional order (q, k, v, attn_mask, dropout_p, is_causal, scale), told
    apart by a fourth argument that is not a layout string.  SDPA tensors are
    (..., H, N, D): 4-D is HND, 3-D (H, N, D) gets a batch of one.  A mask or
    a nonzero dropout raises NotImplementedError, which a caller can catch to
    fall back to the original function (the pages' advice for unsupported
    calls); grouped K/V heads need no enable_gqa."""
    if not isinstance(tensor_layout, str):
        # SDPA's positional order: (q, k, v, attn_mask, dropout_p, is_causal, scale)
        attn_mask, dropout_p, is_causal = tensor_layout, is_causal, sm_scale
        scale = None if isinstance(return_lse, bool) else return_lse      # seventh positional, if given
        tensor_layout, sm_scale, return_lse = "HND", None, False
        dropout_p = 0.0 if dropout_p is False else dropout_p
        is_causal = bool(is_causal) if is_causal is not None else False
    if attn_mask is not None:
        raise NotImplementedError("sageattn does not take an attention mask (use is_causal)")
    if dropout_p:
        raise NotImplementedError("sageattn is a forward without dropout (dropout_p must be 0)")
    if scale is not None:
        if sm_scale is not None and sm_scale != scale:
            raise ValueError("give sm_scale or scale, not both")
        sm_scale = scale
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have the same dtype (deployment guide sec. 4.1)")
    if not (q.device == k.device == v.device) or q.device.type != "cuda":
        raise ValueError("q, k, v must be on the same GPU")
    if q.dim() == 3 and k.dim() == 3 and v.dim() == 3 and tensor_layout == "HND":
        res = sageattn(q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), "HND", is_causal, sm_scale, return_lse,
                       qk_quant_gran=qk_quant_gran, pv_accum_dtype=pv_accum_dtype, smooth_k=smooth_k,
                       smooth_v=smooth_v, v_dtype=v_dtype, kv_splits=kv_splits)
        return (res[0][0], res[1][0]) if return_lse else res[0]
    auto_kv_splits(1, 1, 1, 1, 1, is_causal, kv_splits)          # rejects a bad request before any work
    gq, gk = _geometry(q, tensor_layout, None, None), _geometry(k, tensor_layout, None, None)
    fuse = q_fusable(q, gq.B, gq.H, gk.H, gq.N, gq.d, qk_quant_gran, v_dtype, is_causal, False, (gq.sb, gq.sh, gq.sn))
    qk, qv = sage_quant_qkv(q, k, v, tensor_layout=tensor_layout, qk_quant_gran=qk_quant_gran, smooth_k=smooth_k,
                            v_dtype=v_dtype, smooth_v=smooth_v, quantize_q=not fuse)
    n_splits = auto_kv_splits(qk.B, qk.Hq, qk.Hkv, qk.Nq, qk.Nk, is_causal, kv_splits)
    if n_splits > 1:
        return sage_attn_fwd_splitkv(qk, qv, n_splits=n_splits, tensor_layout=tensor_layout, sm_scale=sm_scale,
                                     return_lse=return_lse, pv_accum_dtype=pv_accum_dtype)
    return sage_attn_fwd(qk, qv, tensor_layout=tensor_layout, is_causal=is_causal, sm_scale=sm_scale,
                         return_lse=return_lse, pv_accum_dtype=pv_accum_dtype)


def sageattn_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, is_causal: bool = False,
                    sm_scale: Optional[float] = None, return_lse: bool = False, *,
                    qk_quant_gran: str = "per_thread", pv_accum_dtype: str = "fp32+fp32", smooth_k: bool = True,
                    smooth_v: bool = False, v_dtype: str = "fp8"):
    """Packed variable-length batch: q (total_q, Hq, D), k/v (total_k, Hkv, D);
    cu_seqlens_* int32 [B+1] on the GPU.  Causal masking is per sequence.
    Returns out (total_q, Hq, D) and, with return_lse, fp32 [Hq, total_q]."""
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have the same dtype")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    gq = _geometry(q, "NHD", cu_seqlens_q, max_seqlen_q)
    fuse = q_fusable(q, gq.B, gq.H, k.shape[1] if k.dim() == 3 else gq.H, gq.N, gq.d, qk_quant_gran, v_dtype,
                     is_causal, True, (gq.sb, gq.sh, gq.sn))
    qk, qv = sage_quant_qkv(q, k, v, qk_quant_gran=qk_quant_gran, smooth_k=smooth_k, v_dtype=v_dtype,
                            smooth_v=smooth_v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
                            max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k, quantize_q=not fuse)
    return sage_attn_varlen_fwd(qk, qv, cu_seqlens_q, cu_seqlens_k, q.shape[0], is_causal=is_causal,
                                sm_scale=sm_scale, return_lse=return_lse, pv_accum_dtype=pv_accum_dtype)


def default_sm_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
