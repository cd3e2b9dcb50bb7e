"""Seeded synthetic workloads for the quantized-attention forward.

This module only draws inputs and describes shapes and knobs.  It holds none of
the method's arithmetic, so both the CPU oracle (under ``oracle/``) and the HIP
path may use it without sharing any computation.

Recipe (one NumPy PCG64 generator per workload, seeded with the workload's
seed):

* varlen workloads first draw the sequence lengths with
  ``rng.integers(lo, hi, endpoint=True, size=n_seq)``;
* then Q, K and V, in that order, as ``rng.standard_normal(shape, float32)``
  in the caller's layout (HND = (B, H, N, D), NHD = (B, N, H, D), varlen =
  packed (total_tokens, H, D));
* the video-DiT workload then draws a K bias of shape (H_kv, D) with standard
  deviation 2 (variance 4) and a V bias of shape (H_kv, D) with standard
  deviation 1; each bias is broadcast along the sequence and added in fp32;
* finally every tensor is rounded once, fp32 -> fp16 or bf16, to nearest even.

The five workloads follow the attention shapes named by the SageAttention pages:
the smoke-test shape of the deployment guide (pwwt.cn, section 2 step 3:
B=2, H=8, N=4096, D=128, HND), a decoder-LLM prefill with grouped K/V heads
(deployment guide section 4.1: GQA needs only Hq divisible by Hkv), a
CogVideoX-like video DiT shape (deployment guide section 5.2: 13 latent frames
x 1350 tokens, 48 heads of 64) with biased K and V to exercise smooth_k and
smooth_v (deployment guide section 4.2), and a packed variable-length batch
(deployment guide section 4.2, sageattn_varlen).  Real activations would need
trained model weights, which are not available; these synthetic tensors stand
in for them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int                  # batch (dense) or number of sequences (varlen)
    Hq: int
    Hkv: int
    Nq: int                 # dense sequence length (varlen: max length bound)
    Nk: int
    d: int
    dtype: str              # "fp16" | "bf16"
    layout: str             # "HND" | "NHD" (varlen is always packed token-major)
    causal: bool
    gran: str               # "per_block" | "per_warp" | "per_thread"
    v_dtype: str            # "fp8" | "fp16"
    pv_accum: str           # "fp32" | "fp16" | "fp16+fp32" | "fp32+fp32" ...
    smooth_k: bool
    smooth_v: bool
    return_lse: bool
    seed: int
    varlen: bool = False
    len_lo: int = 0
    len_hi: int = 0
    k_bias_std: float = 0.0
    v_bias_std: float = 0.0


WORKLOADS = {
    # small parity case the oracle finishes in seconds
    "tiny": Workload("tiny", B=1, Hq=2, Hkv=2, Nq=256, Nk=256, d=64, dtype="fp16", layout="HND",
                     causal=False, gran="per_thread", v_dtype="fp16", pv_accum="fp32",
                     smooth_k=True, smooth_v=False, return_lse=False, seed=1),
    # the headline throughput shape
    "b2h8n4096d128": Workload("b2h8n4096d128", B=2, Hq=8, Hkv=8, Nq=4096, Nk=4096, d=128, dtype="fp16",
                              layout="HND", causal=False, gran="per_warp", v_dtype="fp8",
                              pv_accum="fp16+fp32", smooth_k=True, smooth_v=False, return_lse=False, seed=2),
    "gqa_prefill_n8192": Workload("gqa_prefill_n8192", B=1, Hq=32, Hkv=8, Nq=8192, Nk=8192, d=128,
                                  dtype="bf16", layout="NHD", causal=True, gran="per_thread", v_dtype="fp8",
                                  pv_accum="fp32+fp32", smooth_k=True, smooth_v=False, return_lse=True, seed=3),
    "video_dit_n17550": Workload("video_dit_n17550", B=1, Hq=48, Hkv=48, Nq=17550, Nk=17550, d=64,
                                 dtype="fp16", layout="HND", causal=False, gran="per_thread", v_dtype="fp8",
                                 pv_accum="fp32+fp32", smooth_k=True, smooth_v=True, return_lse=False, seed=4,
                                 k_bias_std=2.0, v_bias_std=1.0),
    "varlen16_h16": Workload("varlen16_h16", B=16, Hq=16, Hkv=16, Nq=4096, Nk=4096, d=128, dtype="fp16",
                             layout="NHD", causal=True, gran="per_thread", v_dtype="fp8", pv_accum="fp32+fp32",
                             smooth_k=True, smooth_v=False, return_lse=False, seed=5,
                             varlen=True, len_lo=128, len_hi=4096),
    # the WSL page's timing comparison with torch's attention (section 5: batch 8, 32 heads, 2048 tokens,
    # head_dim 128, fp16), run with sageattn's default knobs
    "wsl_sdpa_b8h32n2048d128": Workload("wsl_sdpa_b8h32n2048d128", B=8, Hq=32, Hkv=32, Nq=2048, Nk=2048, d=128,
                                        dtype="fp16", layout="HND", causal=False, gran="per_thread",
                                        v_dtype="fp8", pv_accum="fp32+fp32", smooth_k=True, smooth_v=False,
                                        return_lse=False, seed=6),
    # few queries against a long context ([guide] sec. 4.1: q and k/v lengths may differ): 16 query rows per
    # (batch, head) against 32 768 keys, grouped K/V heads, for the split-KV forward
    "decode_gqa_b4_q16_k32768": Workload("decode_gqa_b4_q16_k32768", B=4, Hq=32, Hkv=8, Nq=16, Nk=32768, d=128,
                                         dtype="bf16", layout="NHD", causal=False, gran="per_thread",
                                         v_dtype="fp8", pv_accum="fp32+fp32", smooth_k=True, smooth_v=False,
                                         return_lse=False, seed=7),
}

# the order in which the workloads are listed as configurations
WORKLOAD_ORDER = ["tiny", "b2h8n4096d128", "gqa_prefill_n8192", "video_dit_n17550", "varlen16_h16"]

TORCH_DTYPE = {"fp16": torch.float16, "bf16": torch.bfloat16}


def round_to(x32: np.ndarray, dtype: str) -> torch.Tensor:
    """fp32 array -> fp16/bf16 CPU tensor, rounding to nearest even."""
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(TORCH_DTYPE[dtype])


def make_inputs(w: Workload, scale_down: Optional[dict] = None) -> dict:
    """Draw the workload's tensors.  ``scale_down`` may override shape fields
    (B, Hq, Hkv, Nq, Nk, d, len_hi) to get a smaller case with the same recipe.

    Returns a dict with CPU tensors ``q``, ``k``, ``v`` (fp16/bf16, caller's
    layout), plus ``cu_seqlens`` (int32, varlen only) and the resolved shape.
    """
    if scale_down:
        w = dataclasses.replace(w, **scale_down)
    rng = np.random.default_rng(w.seed)
    out = {"workload": w}
    if w.varlen:
        lens = rng.integers(w.len_lo, w.len_hi, endpoint=True, size=w.B).astype(np.int64)
        cu = np.zeros(w.B + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lens)
        total = int(cu[-1])
        qshape = (total, w.Hq, w.d)
        kshape = (total, w.Hkv, w.d)
        out["cu_seqlens"] = torch.from_numpy(cu.astype(np.int32))
        out["lens"] = lens
        out["max_seqlen"] = int(lens.max())
    elif w.layout == "HND":
        qshape = (w.B, w.Hq, w.Nq, w.d)
        kshape = (w.B, w.Hkv, w.Nk, w.d)
    elif w.layout == "NHD":
        qshape = (w.B, w.Nq, w.Hq, w.d)
        kshape = (w.B, w.Nk, w.Hkv, w.d)
    else:
        raise ValueError(f"unknown layout {w.layout}")
    q = rng.standard_normal(qshape, dtype=np.float32)
    k = rng.standard_normal(kshape, dtype=np.float32)
    v = rng.standard_normal(kshape, dtype=np.float32)
    if w.k_bias_std or w.v_bias_std:
        kb = (w.k_bias_std * rng.standard_normal((w.Hkv, w.d))).astype(np.float32)
        vb = (w.v_bias_std * rng.standard_normal((w.Hkv, w.d))).astype(np.float32)
        if w.varlen or w.layout == "NHD":
            k += kb[None, :, :] if w.varlen else kb[None, None, :, :]
            v += vb[None, :, :] if w.varlen else vb[None, None, :, :]
        else:
            k += kb[None, :, None, :]
            v += vb[None, :, None, :]
    out["q"] = round_to(q, w.dtype)
    out["k"] = round_to(k, w.dtype)
    out["v"] = round_to(v, w.dtype)
    return out


def attention_ops(w: Workload, lens=None) -> float:
    """Operation count used for TOPS: 4 * Nq * Nk * d per (batch, head),
    halved for causal attention; summed over sequences for varlen."""
    if w.varlen:
        assert lens is not None
        per = float(np.sum(np.asarray(lens, dtype=np.float64) ** 2))
        ops = 4.0 * w.Hq * per * w.d
    else:
        ops = 4.0 * w.B * w.Hq * float(w.Nq) * float(w.Nk) * w.d
    return ops / 2.0 if w.causal else ops


def make_merge_inputs(seed: int, S: int, B: int, H: int, N: int, d: int, dtype: str = "fp16",
                      layout: str = "HND", empty_part_frac: float = 0.05, empty_row_frac: float = 0.01) -> dict:
    """Seeded inputs of the merge of partial attention results.

    Recipe: one PCG64 generator seeded with ``seed`` draws, in this order,
    the S partial outputs as standard normals in fp32 (shape (S, B, H, N, d)
    for HND, (S, B, N, H, d) for NHD), the S log-sum-exp values per row as
    normals with mean 8 and standard deviation 2 (fp32, (S, B, H, N)), a
    uniform [0, 1) draw per (part, row) that marks the part empty (LSE =
    -inf, it saw no key) below ``empty_part_frac``, and a uniform draw per row
    that marks the whole row empty below ``empty_row_frac``; the outputs are
    then rounded once to fp16/bf16 (nearest even).  An empty part's output is
    zero, as the forward writes it."""
    rng = np.random.default_rng(seed)
    shape = (S, B, H, N, d) if layout == "HND" else (S, B, N, H, d)
    o = rng.standard_normal(shape, dtype=np.float32)
    lse = (8.0 + 2.0 * rng.standard_normal((S, B, H, N))).astype(np.float32)
    empty = rng.random((S, B, H, N)) < empty_part_frac
    empty |= (rng.random((B, H, N)) < empty_row_frac)[None]
    lse[empty] = -np.inf
    mask = empty if layout == "HND" else np.transpose(empty, (0, 1, 3, 2))
    o[mask] = 0.0
    return {"out_parts": round_to(o, dtype), "lse_parts": torch.from_numpy(lse), "layout": layout,
            "dtype": dtype, "shape": (S, B, H, N, d)}
