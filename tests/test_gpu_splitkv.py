"""GPU parity of the split-KV forward (few queries, many keys; needs an MI355X).

sage_attn_fwd_splitkv against the oracle's split emulation
(oracle.reference_forward_splitkv) on the same seeded inputs: per element
|gpu - oracle| <= 2e-3 + 1 output ulp (the dense forward's bound) + the
oracle's merged allowance + 3e-5 * the largest range output of the row (the
merge's fp32 weights: range LSEs of magnitude below ~50 carry fp32 rounding
of a few 1e-6, and each weight's exp adds an ulp), and cosine >= 0.9999; the
merged LSE within 2e-3 + the LSE allowance.  The ranges' partial outputs are
kept in fp32, so no rounding happens before the final one.  One range is bit-identical to
sage_attn_fwd.  On a decode-like shape (16 queries, 16 384 keys) the result is
within the method's tolerance of exact attention (cosine >= 0.999).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import quantized_attention_smooth_amd as sage
from parity_utils import COS_EMU, COS_EXACT, EXP_BAND, cosine, out_ulp

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, layout, gran, smooth_v, n_splits, lse, V
    (1, 8, 2, 4, 4133, 128, "fp16", "HND", "per_thread", False, 5, True, "fp8"),
    (2, 4, 4, 33, 3000, 64, "bf16", "NHD", "per_warp", True, 3, True, "fp8"),
    (1, 2, 2, 300, 1000, 96, "fp16", "HND", "per_block", False, 7, False, "fp8"),
    (1, 4, 1, 1, 640, 128, "bf16", "HND", "per_thread", False, 64, True, "fp8"),
    (1, 4, 2, 8, 2100, 128, "fp16", "HND", "per_thread", False, 4, True, "fp16"),
    (2, 2, 2, 40, 900, 64, "bf16", "NHD", "per_warp", True, 3, False, "fp16"),
]


def _quantize(q, k, v, layout, gran, smooth_v, v_dtype="fp8"):
    return sage.sage_quant_qkv(q, k, v, tensor_layout=layout, qk_quant_gran=gran, smooth_k=True, v_dtype=v_dtype,
                               smooth_v=smooth_v)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}_{}_{}_sv{}_S{}_V{}".format(
    *c[:11], c[12]))
def test_splitkv_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, d, dtype, layout, gran, smooth_v, ns, want_lse, v_dtype = case
    print(f"[gpu-case] split-KV {case} seed 2", flush=True)
    w = workloads.WORKLOADS["b2h8n4096d128"]
    inp = workloads.make_inputs(w, {"B": B, "Hq": Hq, "Hkv": Hkv, "Nq": Nq, "Nk": Nk, "d": d, "dtype": dtype,
                                    "layout": layout})
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    qk, qv = _quantize(q, k, v, layout, gran, smooth_v, v_dtype)
    res = sage.sage_attn_fwd_splitkv(qk, qv, n_splits=ns, tensor_layout=layout, return_lse=want_lse)
    out, lse = res if want_lse else (res, None)
    torch.cuda.synchronize()
    ref = oracle.reference_forward_splitkv(*(inp[x].float().numpy() for x in ("q", "k", "v")), dtype=dtype,
                                           n_splits=ns, layout=layout, gran=gran, smooth_v=smooth_v,
                                           v_dtype=v_dtype, exp_band=EXP_BAND)
    got = out.float().cpu().numpy()
    if layout == "NHD":
        got = got.transpose(0, 2, 1, 3)
    for b in range(B):
        r = ref["out"][b]
        tol = 2e-3 + out_ulp(r, dtype) + ref["allow"][b] + 3e-5 * ref["parts_scale"][b][..., None]
        diff = np.abs(got[b] - r)
        assert (diff <= tol).all(), f"batch {b}: {(diff > tol).sum()} outputs off, worst {diff.max():.3g}"
        assert cosine(got[b], r) >= COS_EMU
        if want_lse:
            assert np.all(np.abs(lse[b].cpu().numpy() - ref["lse"][b]) <= 2e-3 + ref["lse_allow"][b])


def test_one_range_is_bit_identical_to_attn_fwd():
    print("[gpu-case] split-KV one range vs sage_attn_fwd: B1 H4 Nq200 Nk700 d128 fp16 seed 2", flush=True)
    w = workloads.WORKLOADS["b2h8n4096d128"]
    inp = workloads.make_inputs(w, {"B": 1, "Hq": 4, "Hkv": 4, "Nq": 200, "Nk": 700})
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    qk, qv = _quantize(q, k, v, "HND", "per_warp", False)
    o1, l1 = sage.sage_attn_fwd(qk, qv, return_lse=True)
    o2, l2 = sage.sage_attn_fwd_splitkv(qk, qv, n_splits=1, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_shape_close_to_exact_attention():
    print("[gpu-case] split-KV decode: B1 Hq16 Hkv4 Nq16 Nk16384 d128 bf16 NHD, automatic splits, seed 3", flush=True)
    w = workloads.WORKLOADS["gqa_prefill_n8192"]
    inp = workloads.make_inputs(w, {"B": 1, "Hq": 16, "Hkv": 4, "Nq": 16, "Nk": 16384})
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    qk, qv = _quantize(q, k, v, "NHD", "per_thread", False)
    out, lse = sage.sage_attn_fwd_splitkv(qk, qv, tensor_layout="NHD", return_lse=True)
    torch.cuda.synchronize()
    ex = oracle.exact_forward(*(inp[x].float().numpy() for x in ("q", "k", "v")), layout="NHD")
    got = out.float().cpu().numpy()[0].transpose(1, 0, 2)
    assert cosine(got, ex["out"][0]) >= COS_EXACT
    assert np.abs(lse.cpu().numpy()[0] - ex["lse"][0]).max() < 0.05


@pytest.mark.parametrize("nq", [1, 16, 100, 128])
def test_packed_gqa_rows_equal_repeated_kv(nq):
    """Few queries with grouped K/V heads run with the rows of a group packed
    into one workgroup; every row's arithmetic is unchanged, so the result is
    bit-identical to the same heads with K/V repeated per query head (which is
    not packed)."""
    print(f"[gpu-case] packed GQA rows: B2 Hq8 Hkv2 Nq{nq} Nk1000 d128 fp16 per_thread seed 2", flush=True)
    w = workloads.WORKLOADS["b2h8n4096d128"]
    inp = workloads.make_inputs(w, {"B": 2, "Hq": 8, "Hkv": 2, "Nq": nq, "Nk": 1000})
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    kr, vr = (t.repeat_interleave(4, dim=1).contiguous() for t in (k, v))
    outs = []
    for kk, vv in ((k, v), (kr, vr)):
        qk, qv = _quantize(q, kk, vv, "HND", "per_thread", False)
        outs.append(sage.sage_attn_fwd(qk, qv, return_lse=True))
        outs.append(sage.sage_attn_fwd_splitkv(qk, qv, n_splits=3, return_lse=True))
    torch.cuda.synchronize()
    for i in (0, 1):
        assert torch.equal(outs[i][0].view(torch.int16), outs[i + 2][0].view(torch.int16))
        assert torch.equal(outs[i][1], outs[i + 2][1])


def test_sageattn_kv_splits_matches_oracle():
    """sageattn(..., kv_splits="auto") on a decode shape equals the oracle's
    split emulation with the number of ranges auto_kv_splits picks."""
    print("[gpu-case] sageattn kv_splits=auto: B2 Hq8 Hkv8 Nq8 Nk5000 d64 fp16 HND seed 2", flush=True)
    w = workloads.WORKLOADS["b2h8n4096d128"]
    inp = workloads.make_inputs(w, {"B": 2, "Hq": 8, "Hkv": 8, "Nq": 8, "Nk": 5000, "d": 64})
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    out = sage.sageattn(q, k, v, kv_splits="auto")
    torch.cuda.synchronize()
    ns = sage.auto_kv_splits(2, 8, 8, 8, 5000, False)
    assert ns > 1
    ref = oracle.reference_forward_splitkv(*(inp[x].float().numpy() for x in ("q", "k", "v")), dtype="fp16",
                                           n_splits=ns, exp_band=EXP_BAND)
    got = out.float().cpu().numpy()
    for b in range(2):
        r = ref["out"][b]
        tol = 2e-3 + out_ulp(r, "fp16") + ref["allow"][b] + 3e-5 * ref["parts_scale"][b][..., None]
        assert (np.abs(got[b] - r) <= tol).all()
    with pytest.raises(NotImplementedError):
        sage.sageattn(q, k, v, is_causal=True, kv_splits=2)


def test_sageattn_splits_by_default_only_when_the_gpu_is_not_filled():
    """sageattn's default (kv_splits="auto") is the split-KV forward on a
    decode shape and the one-pass forward on a shape whose row tiles fill the
    GPU, bit for bit."""
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS["b2h8n4096d128"]
    for shape, split in (({"B": 2, "Hq": 8, "Hkv": 8, "Nq": 8, "Nk": 5000, "d": 64}, True),
                         ({"B": 2, "Hq": 8, "Hkv": 8, "Nq": 4096, "Nk": 1024, "d": 64}, False)):
        print(f"[gpu-case] sageattn default kv_splits on {shape} seed 2", flush=True)
        inp = workloads.make_inputs(w, shape)
        q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
        out = sage.sageattn(q, k, v)
        qk, qv = sage.sage_quant_qkv(q, k, v, qk_quant_gran="per_thread")
        ns = sage.auto_kv_splits(shape["B"], shape["Hq"], shape["Hkv"], shape["Nq"], shape["Nk"], False)
        assert (ns > 1) == split
        ref = sage.sage_attn_fwd_splitkv(qk, qv, n_splits=ns) if split else sage.sage_attn_fwd(qk, qv)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_one_range_fp16_v_is_bit_identical_to_attn_fwd():
    print("[gpu-case] split-KV fp16 V one range vs sage_attn_fwd: B1 H4 Nq200 Nk700 d128 bf16 seed 2", flush=True)
    w = workloads.WORKLOADS["b2h8n4096d128"]
    inp = workloads.make_inputs(w, {"B": 1, "Hq": 4, "Hkv": 4, "Nq": 200, "Nk": 700, "dtype": "bf16"})
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    qk, qv = _quantize(q, k, v, "HND", "per_thread", False, "fp16")
    o1, l1 = sage.sage_attn_fwd(qk, qv, return_lse=True)
    o2, l2 = sage.sage_attn_fwd_splitkv(qk, qv, n_splits=1, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
