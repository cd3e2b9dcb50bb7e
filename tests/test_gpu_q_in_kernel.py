"""Attention with Q in its input precision, quantized by the attention kernel
itself, against the same call on the INT8 Q of the quantize pass (needs an
MI355X).

The kernel forms the same codes and scales as the quantize pass (one shared
arithmetic helper), so the two calls must give the same output and LSE bits;
the K/V-only quantize call must write the same K and V operands as the full
one.  The cases cover the three granularities, ragged row counts (a partial
last tile), head_dim below the padded width, packed grouped heads, causal
masks, varlen batches and the split-KV forward; the sageattn entry takes this
path on its own where it is available.
"""
import dataclasses

import pytest
import torch

import workloads
import quantized_attention_smooth_amd as sage

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, layout, gran, causal, smooth_v, lse
    (2, 4, 4, 1000, 777, 128, "fp16", "HND", "per_warp", False, False, True),
    (1, 8, 2, 333, 1200, 72, "bf16", "NHD", "per_thread", True, True, True),
    (1, 4, 4, 700, 700, 96, "fp16", "HND", "per_block", False, False, False),
    (1, 4, 4, 600, 650, 128, "bf16", "NHD", "per_block", True, False, True),
    (1, 8, 2, 64, 2000, 128, "bf16", "HND", "per_warp", False, False, True),      # packed rows, Nq % 32 == 0
    (1, 8, 2, 128, 900, 128, "fp16", "NHD", "per_block", False, True, True),      # packed rows, Nq % 128 == 0
    (1, 16, 4, 17, 1500, 128, "fp16", "HND", "per_thread", False, False, True),   # packed rows, ragged
]

FIELDS_K = ("k8", "k_scale", "k_mean")
FIELDS_V = ("vt", "v_scale", "v_mean")


def _same_kv(a, b, what):
    (qa, va), (qb, vb) = a, b
    for f in FIELDS_K:
        x, y = getattr(qa, f), getattr(qb, f)
        assert (x is None) == (y is None), (what, f)
        if x is not None:
            assert torch.equal(x, y), (what, f)
    for f in FIELDS_V:
        x, y = getattr(va, f), getattr(vb, f)
        assert (x is None) == (y is None), (what, f)
        if x is not None:
            assert torch.equal(x, y), (what, f)


def _bits_equal(x, y):
    return torch.equal(x.contiguous().view(torch.int16), y.contiguous().view(torch.int16))


def _case_id(c):
    return "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}_{}_{}_causal{}_sv{}_lse{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_q_in_kernel_matches_int8_q(case):
    B, Hq, Hkv, Nq, Nk, d, dtype, layout, gran, causal, smooth_v, lse = case
    print(f"[gpu-case] Q quantized in the attention kernel: {_case_id(case)} seed 2", flush=True)
    w = workloads.WORKLOADS["b2h8n4096d128"]
    inp = workloads.make_inputs(w, {"B": B, "Hq": Hq, "Hkv": Hkv, "Nq": Nq, "Nk": Nk, "d": d, "dtype": dtype,
                                    "layout": layout})
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    g = sage.api._geometry(q, layout, None, None)
    assert sage.q_fusable(q, B, Hq, Hkv, Nq, d, gran, "fp8", causal, False, (g.sb, g.sh, g.sn))
    kw = dict(tensor_layout=layout, qk_quant_gran=gran, smooth_k=True, v_dtype="fp8", smooth_v=smooth_v)
    ref = sage.sage_quant_qkv(q, k, v, **kw)
    fused = sage.sage_quant_qkv(q, k, v, quantize_q=False, **kw)
    assert fused[0].q8 is None and fused[0].q is not None
    _same_kv(ref, fused, "K/V operands")
    akw = dict(tensor_layout=layout, is_causal=causal, return_lse=lse)
    a = sage.sage_attn_fwd(*ref, **akw)
    b = sage.sage_attn_fwd(*fused, **akw)
    torch.cuda.synchronize()
    if lse:
        assert _bits_equal(a[0], b[0])
        assert torch.equal(a[1], b[1])
    else:
        assert _bits_equal(a, b)
    if not causal:
        print(f"[gpu-case]   split-KV, 3 ranges", flush=True)
        sa = sage.sage_attn_fwd_splitkv(*ref, n_splits=3, tensor_layout=layout, return_lse=True)
        sb = sage.sage_attn_fwd_splitkv(*fused, n_splits=3, tensor_layout=layout, return_lse=True)
        torch.cuda.synchronize()
        assert _bits_equal(sa[0], sb[0]) and torch.equal(sa[1], sb[1])


@pytest.mark.parametrize("gran", ["per_thread", "per_warp", "per_block"])
def test_q_in_kernel_varlen(gran):
    w = dataclasses.replace(workloads.WORKLOADS["varlen16_h16"], B=5, Hq=4, Hkv=2, len_lo=1, len_hi=700, seed=41)
    print(f"[gpu-case] Q quantized in the varlen attention kernel: {gran} seed {w.seed}", flush=True)
    inp = workloads.make_inputs(w)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    cu, ms = inp["cu_seqlens"].to(DEV), inp["max_seqlen"]
    kw = dict(qk_quant_gran=gran, smooth_k=True, v_dtype="fp8", smooth_v=False, cu_seqlens_q=cu, cu_seqlens_k=cu,
              max_seqlen_q=ms, max_seqlen_k=ms)
    ref = sage.sage_quant_qkv(q, k, v, **kw)
    fused = sage.sage_quant_qkv(q, k, v, quantize_q=False, **kw)
    total = q.shape[0]
    for causal in (True, False):
        a = sage.sage_attn_varlen_fwd(*ref, cu, cu, total, is_causal=causal, return_lse=True)
        b = sage.sage_attn_varlen_fwd(*fused, cu, cu, total, is_causal=causal, return_lse=True)
        torch.cuda.synchronize()
        assert _bits_equal(a[0], b[0]), causal
        assert torch.equal(a[1], b[1]), causal


def test_q_in_kernel_bf16_input_fp16_output():
    """Q's element type is the call's input type, independent of the output's."""
    w = workloads.WORKLOADS["b2h8n4096d128"]
    print("[gpu-case] Q quantized in the attention kernel: bf16 Q/K/V, fp16 out, per_block", flush=True)
    inp = workloads.make_inputs(w, {"B": 1, "Hq": 4, "Hkv": 4, "Nq": 520, "Nk": 600, "dtype": "bf16"})
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    kw = dict(tensor_layout="HND", qk_quant_gran="per_block", smooth_k=True, v_dtype="fp8")
    ref = sage.sage_quant_qkv(q, k, v, **kw)
    fused = sage.sage_quant_qkv(q, k, v, quantize_q=False, **kw)
    outs = []
    for qk, qv in (ref, fused):
        out = torch.empty(q.shape, dtype=torch.float16, device=DEV)
        outs.append(sage.sage_attn_fwd(qk, qv, tensor_layout="HND", out=out))
    torch.cuda.synchronize()
    assert _bits_equal(outs[0], outs[1])


def test_sageattn_quantizes_q_in_the_kernel_when_it_can():
    w = workloads.WORKLOADS["b2h8n4096d128"]
    print("[gpu-case] sageattn on b2h8n4096d128 (per_warp, fp16 HND): Q in the kernel", flush=True)
    inp = workloads.make_inputs(w, {"Nq": 1024, "Nk": 1024})
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    g = sage.api._geometry(q, "HND", None, None)
    assert sage.q_fusable(q, g.B, g.H, g.H, g.N, g.d, w.gran, "fp8", False, False, (g.sb, g.sh, g.sn))
    out = sage.sageattn(q, k, v, "HND", False, qk_quant_gran=w.gran, kv_splits=None)
    ref = sage.sage_attn_fwd(*sage.sage_quant_qkv(q, k, v, tensor_layout="HND", qk_quant_gran=w.gran,
                                                  smooth_k=True, v_dtype="fp8"))
    torch.cuda.synchronize()
    assert _bits_equal(out, ref)
    # FP16 V runs the other kernel, which reads INT8 Q: the call quantizes Q first
    assert not sage.q_fusable(q, g.B, g.H, g.H, g.N, g.d, w.gran, "fp16", False, False, (g.sb, g.sh, g.sn))
    qk, qv = sage.sage_quant_qkv(q, k, v, tensor_layout="HND", qk_quant_gran=w.gran, v_dtype="fp16",
                                 quantize_q=False)
    with pytest.raises(NotImplementedError, match="input precision"):
        sage.sage_attn_fwd(qk, qv, tensor_layout="HND")


@pytest.mark.parametrize("quantize_q", [True, False])
def test_quant_plan_matches_the_call(quantize_q):
    """QuantQKVPlan (outputs and parameter blocks made once) writes what
    sage_quant_qkv writes, on every run into the same buffers."""
    w = workloads.WORKLOADS["gqa_prefill_n8192"]
    print(f"[gpu-case] quantize plan: gqa shape scaled down, quantize_q={quantize_q}", flush=True)
    inp = workloads.make_inputs(w, {"Nq": 700, "Nk": 700})
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    kw = dict(tensor_layout=w.layout, qk_quant_gran=w.gran, smooth_k=True, v_dtype="fp8", smooth_v=True,
              quantize_q=quantize_q)
    ref = sage.sage_quant_qkv(q, k, v, **kw)
    plan = sage.QuantQKVPlan(q, k, v, **kw)
    for _ in range(2):
        got = plan.run()
        torch.cuda.synchronize()
        _same_kv(ref, got, "plan")
        if quantize_q:
            assert torch.equal(ref[0].q8, got[0].q8) and torch.equal(ref[0].q_scale, got[0].q_scale)
        else:
            assert got[0].q8 is None and got[0].q is q
