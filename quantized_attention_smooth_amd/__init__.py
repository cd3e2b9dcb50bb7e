"""MI355X (gfx950) quantized attention forward, SageAttention style.

out = softmax(Q K^T * sm_scale) V with smooth_k, INT8 Q/K (per-block / per-warp
/ per-thread fp32 scales), INT8 MFMA QK^T, online softmax, FP8 (or FP16/BF16)
P.V with fp32 accumulation, FP16/BF16 output and optional LSE.  The compute
lives in libsage.so (hand-written HIP for gfx950, C ABI in include/sage.h);
this package only marshals arguments.
"""
from .api import (QuantQK, QuantQKVPlan, QuantV, padded_head_dim, sage_attn_fwd, sage_attn_fwd_splitkv, sage_attn_varlen_fwd,
                  sage_debug_qk_scores, sage_merge_states, sage_quant_qk, sage_quant_qkv, sage_quant_qkv_noalloc,
                  sage_quant_v, sageattn, sageattn_varlen, splitkv_plan, workspace_bytes, auto_kv_splits, q_fusable)
from ._abi import LIB_PATH, SageError, load as load_library

__all__ = [
    "QuantQK", "QuantQKVPlan", "QuantV", "padded_head_dim", "sage_attn_fwd", "sage_attn_varlen_fwd", "sage_debug_qk_scores",
    "sage_merge_states", "sage_attn_fwd_splitkv", "splitkv_plan", "sage_quant_qk", "sage_quant_qkv",
    "sage_quant_qkv_noalloc", "sage_quant_v", "sageattn", "auto_kv_splits", "q_fusable", "sageattn_varlen",
    "workspace_bytes", "LIB_PATH",
    "SageError", "load_library",
]
