"""ctypes mirror of include/sage.h and the loader for libsage.so.

Argument marshalling only: every step of the forward runs in the HIP kernels
of libsage.so.  There is no fallback: if the library is missing, importing the
entry points raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsage.so")

SAGE_OK, SAGE_EINVAL, SAGE_EUNSUPPORTED, SAGE_EHIP = 0, -1, -2, -3
SAGE_F16, SAGE_BF16 = 0, 1
SAGE_HND, SAGE_NHD = 0, 1
SAGE_PER_BLOCK, SAGE_PER_WARP, SAGE_PER_THREAD = 0, 1, 2
SAGE_V_FP8, SAGE_V_FP16 = 0, 1
SAGE_ACC_FP32, SAGE_ACC_FP16, SAGE_ACC_FP16_FP32, SAGE_ACC_FP32_FP32 = 0, 1, 2, 3
SAGE_QUANT_SCRATCH_BYTES = 16 << 20

VP = ctypes.c_void_p
I = ctypes.c_int
I64 = ctypes.c_int64
SZ = ctypes.c_size_t


class QuantQKParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", SZ), ("q", VP), ("k", VP), ("dtype", I),
        ("B", I), ("Hq", I), ("Hkv", I), ("Nq", I), ("Nk", I), ("d", I),
        ("q_stride_b", I64), ("q_stride_h", I64), ("q_stride_n", I64),
        ("k_stride_b", I64), ("k_stride_h", I64), ("k_stride_n", I64),
        ("cu_seqlens_q", VP), ("cu_seqlens_k", VP), ("gran", I), ("smooth_k", I),
        ("q8", VP), ("q_scale", VP), ("k8", VP), ("k_scale", VP), ("k_mean", VP),
        ("workspace", VP), ("workspace_bytes", SZ),
    ]


class QuantVParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", SZ), ("v", VP), ("dtype", I),
        ("B", I), ("Hkv", I), ("Nk", I), ("d", I),
        ("v_stride_b", I64), ("v_stride_h", I64), ("v_stride_n", I64),
        ("cu_seqlens_k", VP), ("v_dtype", I), ("smooth_v", I),
        ("vt", VP), ("v_scale", VP), ("v_mean", VP), ("workspace", VP), ("workspace_bytes", SZ),
    ]


class AttnParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", SZ), ("q8", VP), ("q_scale", VP), ("k8", VP), ("k_scale", VP), ("k_mean", VP),
        ("vt", VP), ("v_scale", VP), ("v_mean", VP),
        ("B", I), ("Hq", I), ("Hkv", I), ("Nq", I), ("Nk", I), ("d", I),
        ("gran", I), ("v_dtype", I), ("pv_accum", I), ("is_causal", I), ("sm_scale", ctypes.c_float),
        ("in_dtype", I), ("out", VP), ("out_dtype", I),
        ("o_stride_b", I64), ("o_stride_h", I64), ("o_stride_n", I64), ("lse", VP),
        ("q", VP), ("q_stride_b", I64), ("q_stride_h", I64), ("q_stride_n", I64),
    ]


class AttnVarlenParams(ctypes.Structure):
    _fields_ = [("base", AttnParams), ("cu_seqlens_q", VP), ("cu_seqlens_k", VP), ("total_q", I)]


class MergeParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", SZ), ("n_parts", I), ("dtype", I), ("B", I), ("H", I), ("N", I), ("d", I),
        ("parts", VP), ("ps_s", I64), ("ps_b", I64), ("ps_h", I64), ("ps_n", I64), ("lse_parts", VP),
        ("out", VP), ("o_stride_b", I64), ("o_stride_h", I64), ("o_stride_n", I64), ("lse", VP),
    ]


EXPORTS = ["sage_quant_qk", "sage_quant_workspace_size", "sage_quant_v", "sage_quant_qkv",
           "sage_quant_qkv_noalloc_scratch_size", "sage_quant_qkv_noalloc", "sage_attn_fwd",
           "sage_attn_varlen_fwd", "sage_debug_qk_scores", "sage_debug_qk_scores_varlen", "sage_merge_states", "sage_attn_splitkv_workspace_size",
           "sage_attn_fwd_splitkv", "sage_attn_q_fusable", "sage_last_error", "sage_version"]

_lib = None


class SageError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load libsage.so (built by quantized_attention_smooth_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build the HIP library first "
                          "(python -m quantized_attention_smooth_amd.build)")
    L = ctypes.CDLL(path)
    L.sage_quant_qk.argtypes = [ctypes.POINTER(QuantQKParams), VP]
    L.sage_quant_qk.restype = I
    L.sage_quant_v.argtypes = [ctypes.POINTER(QuantVParams), VP]
    L.sage_quant_v.restype = I
    L.sage_quant_qkv.argtypes = [ctypes.POINTER(QuantQKParams), ctypes.POINTER(QuantVParams), VP]
    L.sage_quant_qkv.restype = I
    L.sage_quant_qkv_noalloc.argtypes = [ctypes.POINTER(QuantQKParams), ctypes.POINTER(QuantVParams), VP]
    L.sage_quant_qkv_noalloc.restype = I
    L.sage_quant_qkv_noalloc_scratch_size.argtypes = [I, I, I, I]
    L.sage_quant_qkv_noalloc_scratch_size.restype = SZ
    L.sage_attn_fwd.argtypes = [ctypes.POINTER(AttnParams), VP]
    L.sage_attn_fwd.restype = I
    L.sage_attn_q_fusable.argtypes = [I, I, I, I, I, I, I, I, I]
    L.sage_attn_q_fusable.restype = I
    L.sage_attn_varlen_fwd.argtypes = [ctypes.POINTER(AttnVarlenParams), VP]
    L.sage_attn_varlen_fwd.restype = I
    L.sage_debug_qk_scores.argtypes = [ctypes.POINTER(AttnParams), I, VP, VP]
    L.sage_debug_qk_scores.restype = I
    L.sage_debug_qk_scores_varlen.argtypes = [ctypes.POINTER(AttnVarlenParams), VP, VP]
    L.sage_debug_qk_scores_varlen.restype = I
    L.sage_attn_fwd_splitkv.argtypes = [ctypes.POINTER(AttnParams), I, VP, SZ, VP]
    L.sage_attn_fwd_splitkv.restype = I
    L.sage_attn_splitkv_workspace_size.argtypes = [I, I, I, I, I, I]
    L.sage_attn_splitkv_workspace_size.restype = SZ
    L.sage_merge_states.argtypes = [ctypes.POINTER(MergeParams), VP]
    L.sage_merge_states.restype = I
    L.sage_quant_workspace_size.argtypes = [I, I, I, I]
    L.sage_quant_workspace_size.restype = SZ
    L.sage_last_error.argtypes = []
    L.sage_last_error.restype = ctypes.c_char_p
    L.sage_version.argtypes = []
    L.sage_version.restype = I
    _lib = L
    return L


def check(rc: int) -> None:
    if rc == SAGE_OK:
        return
    msg = load().sage_last_error().decode(errors="replace")
    if rc == SAGE_EINVAL:
        raise ValueError(msg)
    if rc == SAGE_EUNSUPPORTED:
        raise NotImplementedError(msg)
    raise SageError(f"HIP failure: {msg}")
