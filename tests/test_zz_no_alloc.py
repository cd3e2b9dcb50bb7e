"""The no-alloc quantize call (sage_quant_qkv_noalloc, statistics partials in
the library's static device array) against sage_quant_qkv (caller
workspaces), bit for bit, on consecutive calls whose sizes shrink: the second
and third calls reuse the array the first one filled, so a partial left over
from an earlier call would show.  Needs an MI355X."""
import dataclasses

import pytest
import torch

import workloads
import quantized_attention_smooth_amd as sage
from parity_utils import written_quant_outputs

pytestmark = pytest.mark.gpu

FIELDS_QK = ("q8", "q_scale", "k8", "k_scale", "k_mean")
FIELDS_V = ("vt", "v_scale", "v_mean")


def _both(inp, w, v_dtype, smooth_v):
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    kw = dict(qk_quant_gran=w.gran, smooth_k=w.smooth_k, v_dtype=v_dtype, smooth_v=smooth_v)
    if w.varlen:
        cu = inp["cu_seqlens"].to(dev)
        ms = inp["max_seqlen"]
        kw.update(cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=ms, max_seqlen_k=ms)
    else:
        kw.update(tensor_layout=w.layout)
    ref = sage.sage_quant_qkv(q, k, v, **kw)
    got = sage.sage_quant_qkv_noalloc(q, k, v, **kw)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, what, lens=None):
    a = written_quant_outputs(*ref, lens)
    b = written_quant_outputs(*got, lens)
    for f in FIELDS_QK + FIELDS_V:
        x, y = a[f], b[f]
        assert (x is None) == (y is None), (what, f)
        if x is not None:
            assert torch.equal(x, y), (what, f)


def test_noalloc_equals_workspace_call_on_shrinking_calls():
    cases = [
        ("b2h8n4096d128 (fp16 HND per_warp, FP8 V, smooth_v)",
         workloads.WORKLOADS["b2h8n4096d128"], "fp8", True),
        ("B1 Hq4 Hkv2 N333 d64 bf16 NHD per_thread, fp16 V, smooth_v",
         dataclasses.replace(workloads.WORKLOADS["gqa_prefill_n8192"], Hq=4, Hkv=2, Nq=333, Nk=333, d=64, seed=31),
         "fp16", True),
        ("varlen 3 sequences H2 d128 fp16, FP8 V",
         dataclasses.replace(workloads.WORKLOADS["varlen16_h16"], B=3, Hq=2, Hkv=2, len_lo=1, len_hi=200, seed=32),
         "fp8", False),
    ]
    sizes = []
    for name, w, v_dtype, smooth_v in cases:
        print(f"[gpu-case] no-alloc quantize: {name} seed {w.seed}", flush=True)
        inp = workloads.make_inputs(w)
        B = w.B
        N = inp["max_seqlen"] if w.varlen else w.Nk
        need = sage.load_library().sage_quant_qkv_noalloc_scratch_size(B, w.Hkv, N, w.d)
        sizes.append(need)
        ref, got = _both(inp, w, v_dtype, smooth_v)
        _same(ref, got, name, inp["lens"] if w.varlen else None)
    assert sizes[1] < sizes[0] and sizes[2] < sizes[0]


def test_noalloc_rejects_oversize_without_launching():
    print("[gpu-case] no-alloc quantize: oversize request rejected on the host", flush=True)
    dev = torch.device("cuda:0")
    # sizes whose statistics exceed the static array (600 heads of 8 chunks of
    # 256 tokens); the call fails on the host before its first HIP call
    w = dataclasses.replace(workloads.WORKLOADS["b2h8n4096d128"], B=1, Hq=600, Hkv=600, Nq=2048, Nk=2048, seed=33)
    q = torch.zeros((1, 600, 2048, 128), dtype=torch.float16, device=dev)
    need = sage.load_library().sage_quant_qkv_noalloc_scratch_size(1, 600, 2048, 128)
    assert need > 16 << 20
    with pytest.raises(ValueError, match="too large for the no-alloc call"):
        sage.sage_quant_qkv_noalloc(q, q, q, qk_quant_gran=w.gran)
