"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Bit-exact: INT8 Q/K codes, their scales, K/V means, FP8 V codes and scales,
and the int32 QK^T scores.  Within tolerance: outputs and LSE (see
parity_utils).  Every case prints its name, shape and seed first, so that a
failing GPU step can be identified from its last line of output.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import quantized_attention_smooth_amd as sage
from parity_utils import Case, bf16_sum_exact_in_fp64, cosine, sample_rows, scale_down, written_quant_outputs

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


# ------------------------------------------------------------------ tiny workload, everything
def test_tiny_workload_full():
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny"])
    _announce("tiny B1 H2 N256 d64 fp16 per_thread FP16-V seed 1")
    c = Case(inp["workload"], inp).run_gpu(return_lse=True).run_oracle(exact=True)
    c.check_quantized_bitexact()
    c.check_outputs(lse=True)
    # full int32 score dump against the oracle's exact integer scores
    S = sage.sage_debug_qk_scores(c.qk).cpu().numpy()
    ref = oracle.reference_forward(*(inp[x].float().numpy() for x in ("q", "k", "v")), dtype="fp16",
                                   gran="per_thread", v_dtype="fp16", want_scores=True)
    for h in range(2):
        np.testing.assert_array_equal(S[0, h], ref["scores"][0][h])


# ------------------------------------------------------------------ full-size workloads
BIG = ["b2h8n4096d128", "gqa_prefill_n8192", "video_dit_n17550", "varlen16_h16"]


@pytest.fixture(scope="module")
def big_cases():
    return {}


def _big(name, cache):
    if name not in cache:
        w = workloads.WORKLOADS[name]
        _announce(f"workload {name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} N{w.Nq} d{w.d} {w.dtype} {w.layout} "
                  f"causal={w.causal} {w.gran} V={w.v_dtype} seed {w.seed}")
        inp = workloads.make_inputs(w)
        cache[name] = Case(w, inp).run_gpu(return_lse=w.return_lse)
    return cache[name]


@pytest.mark.parametrize("name", BIG)
def test_workload_quantization_bitexact(name, big_cases):
    c = _big(name, big_cases)
    c.run_oracle(attention=False)
    c.check_quantized_bitexact()


@pytest.mark.parametrize("name", ["b2h8n4096d128", "gqa_prefill_n8192", "video_dit_n17550"])
def test_workload_score_checksums(name, big_cases):
    """Row checksums sum_j S_ij and sum_j (j+1) S_ij of the kernel's int32
    scores against the oracle's integer codes (an fp64 GEMM of INT8 codes is
    exact here: |S| < 2^22)."""
    c = _big(name, big_cases)
    if not hasattr(c, "ref"):
        c.run_oracle(attention=False)
    got = sage.sage_debug_qk_scores(c.qk, checksums=True).cpu().numpy().view(np.uint64)
    w = c.w
    grp = w.Hq // w.Hkv
    rows = sample_rows(w.seed, 48)(0, w.Nq)
    for b in range(w.B):
        for h in range(w.Hq):
            q8 = c.ref["q8"][b][h][rows].astype(np.float64)
            k8 = c.ref["k8"][b][h // grp].astype(np.float64)
            S = (q8 @ k8.T).astype(np.int64)
            s1 = S.sum(axis=1).astype(np.uint64)
            s2 = (S * (np.arange(k8.shape[0], dtype=np.int64) + 1)[None, :]).sum(axis=1).astype(np.uint64)
            np.testing.assert_array_equal(got[b, h, rows, 0], s1)
            np.testing.assert_array_equal(got[b, h, rows, 1], s2)


def test_varlen_score_checksums(big_cases):
    """The varlen batch's int32 scores, row checksums per sequence, against
    the oracle's integer codes."""
    c = _big("varlen16_h16", big_cases)
    if not hasattr(c, "ref"):
        c.run_oracle(attention=False)
    cu = c.inp["cu_seqlens"]
    got = sage.sage_debug_qk_scores(c.qk, checksums=True, cu_seqlens_q=cu.cuda(), cu_seqlens_k=cu.cuda(),
                                    total_q=int(cu[-1])).cpu().numpy().view(np.uint64)
    grp = c.w.Hq // c.w.Hkv
    for b in range(c.n_seq()):
        nq = c.ref["q8"][b].shape[1]
        rows = sample_rows(c.w.seed, 16)(b, nq)
        for h in range(c.w.Hq):
            q8 = c.ref["q8"][b][h][rows].astype(np.float64)
            k8 = c.ref["k8"][b][h // grp].astype(np.float64)
            S = (q8 @ k8.T).astype(np.int64)
            s1 = S.sum(axis=1).astype(np.uint64)
            s2 = (S * (np.arange(k8.shape[0], dtype=np.int64) + 1)[None, :]).sum(axis=1).astype(np.uint64)
            np.testing.assert_array_equal(got[h, c.cu_np[b] + rows, 0], s1)
            np.testing.assert_array_equal(got[h, c.cu_np[b] + rows, 1], s2)


@pytest.mark.parametrize("name", BIG)
def test_workload_outputs(name, big_cases):
    c = _big(name, big_cases)
    w = c.w
    c.run_oracle(rows=sample_rows(w.seed, 24 if w.Hq * w.B > 64 else 48), exact=True)
    c_emu, c_ex = c.check_outputs(lse=w.return_lse)
    _announce(f"{name}: cos vs oracle {c_emu:.6f}, vs exact fp64 {c_ex:.6f}")


def test_benchmark_workload_every_row(big_cases):
    """Every output row of the benchmark workload (2 x 8 heads x 4096 rows)
    against the oracle, element by element at the forward's tolerance, and
    against exact fp64 attention by cosine."""
    c = _big("b2h8n4096d128", big_cases)
    _announce("b2h8n4096d128: every row against the oracle and exact fp64 attention (about half a minute on the CPU)")
    c.run_oracle(rows=None, exact=True)
    c_emu, c_ex = c.check_outputs()
    _announce(f"b2h8n4096d128 every row: cos vs oracle {c_emu:.6f}, vs exact fp64 {c_ex:.6f}")


@pytest.mark.parametrize("name", BIG)
def test_benchmark_step_equals_checked_path(name, big_cases):
    """The step bench.py times, in its launch configuration (Q quantized in
    the attention kernel where the call allows it), gives the outputs and LSEs
    of the path checked against the oracle above, bit for bit."""
    import bench
    c = _big(name, big_cases)
    step = bench.make_step(c.w, c.inp)
    res = step()
    out, lse = res if isinstance(res, tuple) else (res, None)
    torch.cuda.synchronize()
    _announce(f"{name}: benchmark step with Q quantized in the {'attention kernel' if step.fuse_q else 'quantize pass'}")
    assert np.array_equal(out.float().cpu().numpy(), c.gpu_out)
    if c.gpu_lse is not None:
        assert np.array_equal(lse.cpu().numpy(), c.gpu_lse)


# ------------------------------------------------------------------ the longest sweep length
@pytest.mark.parametrize("causal", [False, True])
def test_sequence_32k_outputs(causal):
    """N = 32 768, the longest length of the benchmark sweep (1K-32K): two
    heads of the sweep's shape (d = 128, fp16, HND, per_warp, FP8 V, smooth_k),
    quantization bit-exact and sampled rows (tile edges, the middle, the last
    rows) against the oracle."""
    w = dataclasses.replace(workloads.WORKLOADS["b2h8n4096d128"], name="n32768_h2", B=1, Hq=2, Hkv=2, Nq=32768,
                            Nk=32768, causal=causal, return_lse=True, seed=9)
    _announce(f"{w.name}: B1 H2 N32768 d128 fp16 HND causal={causal} per_warp V=fp8 seed 9")
    c = Case(w, workloads.make_inputs(w)).run_gpu(return_lse=True)
    c.run_oracle(rows=sample_rows(w.seed, 24), exact=True)
    c.check_quantized_bitexact()
    c_emu, c_ex = c.check_outputs(lse=True)
    _announce(f"{w.name} causal={causal}: cos vs oracle {c_emu:.6f}, vs exact fp64 {c_ex:.6f}")


# ------------------------------------------------------------------ edge-case matrix
SMALL = [
    # (Nq, Nk, d): ragged tails, Nq != Nk, padded head dims
    (200, 200, 128),
    (130, 300, 64),
    (300, 70, 40),
    (65, 129, 96),
    (1, 1, 16),
]


@pytest.mark.parametrize("gran", ["per_block", "per_warp", "per_thread"])
@pytest.mark.parametrize("v_dtype", ["fp8", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_small_matrix(gran, v_dtype, causal, shape, dtype):
    nq, nk, d = shape
    seed = 100 + nq + nk + d
    _announce(f"small {dtype} Nq{nq} Nk{nk} d{d} {gran} V={v_dtype} causal={causal} seed {seed}")
    base = workloads.WORKLOADS["b2h8n4096d128"]
    w = dataclasses.replace(base, B=2, Hq=4, Hkv=2, Nq=nq, Nk=nk, d=d, dtype=dtype, gran=gran,
                                      v_dtype=v_dtype, causal=causal, smooth_v=(v_dtype == "fp8"), seed=seed,
                                      k_bias_std=1.0, v_bias_std=0.5)
    inp = workloads.make_inputs(w)
    c = Case(w, inp).run_gpu(return_lse=True).run_oracle(exact=True)
    c.check_quantized_bitexact()
    c.check_outputs(lse=True)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_small_matches_oracle(causal):
    base = workloads.WORKLOADS["varlen16_h16"]
    w = dataclasses.replace(base, B=5, Hq=4, Hkv=2, len_lo=1, len_hi=300, causal=causal, seed=77)
    _announce(f"varlen small causal={causal} seed 77")
    inp = workloads.make_inputs(w)
    c = Case(w, inp).run_gpu(return_lse=True).run_oracle(exact=True)
    c.check_quantized_bitexact()
    c.check_outputs(lse=True)


# ------------------------------------------------------------------ bf16 means over wide magnitude spans
@pytest.mark.parametrize("n, e_lo, e_hi, within", [(8, -20, 21, True), (4096, -25, 20, False)])
def test_bf16_means_wide_span(n, e_lo, e_hi, within):
    """bf16 K and V whose columns span 41 (N = 8) or 45 (N = 4096) binades:
    sign * (1 + m/128) * 2^e with e uniform in [e_lo, e_hi).  The K and V means
    (smooth_k, smooth_v) must equal the oracle's correctly rounded means
    (math.fsum) bit for bit.  The first case satisfies the exactness condition
    the library states for bf16 sums (every partial sum exact in fp64); the
    second lies beyond it and is checked as it comes out on this seed."""
    _announce(f"bf16 means, N={n}, exponents [{e_lo}, {e_hi}), seed {70 + n}")
    rng = np.random.default_rng(70 + n)
    shape = (1, 2, n, 64)

    def wide():
        mant = 1.0 + rng.integers(0, 128, size=shape) / 128.0
        x = np.where(rng.random(shape) < 0.5, -1.0, 1.0) * mant * np.exp2(rng.integers(e_lo, e_hi, size=shape))
        t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
        assert np.array_equal(t.float().numpy(), x.astype(np.float32))      # exactly bf16 values
        return t, x.astype(np.float32)

    k, kx = wide()
    v, vx = wide()
    q = torch.randn(shape, generator=torch.Generator().manual_seed(70)).bfloat16()
    cols = [kx[0, h, :, c] for h in range(2) for c in range(64)] + [vx[0, h, :, c] for h in range(2) for c in range(64)]
    assert all(bf16_sum_exact_in_fp64(c) for c in cols) == within
    qk, qv = sage.sage_quant_qkv(q.cuda(), k.cuda(), v.cuda(), smooth_k=True, smooth_v=True, v_dtype="fp16")
    torch.cuda.synchronize()
    for h in range(2):
        np.testing.assert_array_equal(qk.k_mean[0, h].cpu().numpy(), oracle.exact_mean(kx[0, h]))
        np.testing.assert_array_equal(qv.v_mean[0, h].cpu().numpy(), oracle.exact_mean(vx[0, h]))


# ------------------------------------------------------------------ structural invariants (bit-exact)
def _run(q, k, v, **kw):
    out = sage.sageattn(q, k, v, **kw)
    torch.cuda.synchronize()
    return out


def test_hnd_equals_nhd():
    _announce("HND == NHD")
    g = torch.Generator().manual_seed(5)
    q, k, v = (torch.randn(2, 3, 333, 128, generator=g).half().cuda() for _ in range(3))
    a = _run(q, k, v, tensor_layout="HND", is_causal=True, qk_quant_gran="per_thread")
    b = _run(q.transpose(1, 2).contiguous(), k.transpose(1, 2).contiguous(), v.transpose(1, 2).contiguous(),
             tensor_layout="NHD", is_causal=True, qk_quant_gran="per_thread")
    assert torch.equal(a, b.transpose(1, 2))
    # non-contiguous NHD views of the HND tensors give the same result too
    c = _run(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), tensor_layout="NHD", is_causal=True,
             qk_quant_gran="per_thread")
    assert torch.equal(a, c.transpose(1, 2))


def test_gqa_equals_repeated_kv():
    _announce("GQA == repeat_interleave")
    g = torch.Generator().manual_seed(6)
    q = torch.randn(1, 8, 300, 64, generator=g).bfloat16().cuda()
    k = torch.randn(1, 2, 300, 64, generator=g).bfloat16().cuda()
    v = torch.randn(1, 2, 300, 64, generator=g).bfloat16().cuda()
    a, la = _run(q, k, v, return_lse=True)
    b, lb = _run(q, k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1), return_lse=True)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_head_dim_padding_equals_explicit_zero_pad():
    _announce("d=96 == zero-padded 128")
    g = torch.Generator().manual_seed(7)
    q, k, v = (torch.randn(1, 2, 257, 96, generator=g).half().cuda() for _ in range(3))
    a = _run(q, k, v)
    pad = lambda x: torch.nn.functional.pad(x, (0, 32))
    b = _run(pad(q), pad(k), pad(v), sm_scale=1 / math.sqrt(96))
    assert torch.equal(a, b[..., :96])
    assert not b[..., 96:].any()


def test_varlen_equals_per_sequence_dense():
    _announce("varlen == per-sequence dense")
    g = torch.Generator().manual_seed(8)
    lens = [1, 77, 128, 300, 64]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    T = int(cu[-1])
    q, k, v = (torch.randn(T, 4, 128, generator=g).half().cuda() for _ in range(3))
    out, lse = sage.sageattn_varlen(q, k, v, cu.cuda(), cu.cuda(), max(lens), max(lens), is_causal=True,
                                    return_lse=True, smooth_v=True)
    for b, n in enumerate(lens):
        s, e = int(cu[b]), int(cu[b + 1])
        qb, kb, vb = (x[s:e].transpose(0, 1).unsqueeze(0).contiguous() for x in (q, k, v))
        ob, lb = _run(qb, kb, vb, is_causal=True, return_lse=True, smooth_v=True)
        assert torch.equal(out[s:e], ob[0].transpose(0, 1)), b
        assert torch.equal(lse[:, s:e], lb[0]), b


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_sequence_longer_than_max_seqlen_is_cut(causal):
    """A sequence longer than the max_seqlen the calls are given is taken as
    its first max_seqlen tokens (all its padded slot holds): the result equals,
    bit for bit, the same batch with that sequence cut, and the output rows
    past the cut keep what they held."""
    _announce(f"varlen sequence beyond max_seqlen, causal={causal}")
    g = torch.Generator().manual_seed(12)
    lens, max_len = [100, 300, 50], 200
    T = sum(lens)
    q, k, v = (torch.randn(T, 4, 128, generator=g).half().cuda() for _ in range(3))
    cu = torch.tensor([0, 100, 400, 450], dtype=torch.int32).cuda()
    keep = torch.tensor(list(range(0, 300)) + list(range(400, 450))).cuda()
    cu_cut = torch.tensor([0, 100, 300, 350], dtype=torch.int32).cuda()
    qk, qv = sage.sage_quant_qkv(q, k, v, cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=max_len,
                                 max_seqlen_k=max_len, smooth_v=True)
    out = torch.full((T, 4, 128), float("nan"), dtype=torch.float16, device="cuda")
    out, lse = sage.sage_attn_varlen_fwd(qk, qv, cu, cu, T, is_causal=causal, return_lse=True, out=out)
    ref, ref_lse = sage.sageattn_varlen(q[keep], k[keep], v[keep], cu_cut, cu_cut, max_len, max_len,
                                        is_causal=causal, return_lse=True, smooth_v=True)
    torch.cuda.synchronize()
    assert torch.equal(out[keep], ref)
    assert torch.equal(lse[:, keep], ref_lse)
    assert torch.isnan(out[300:400]).all()


def test_deterministic():
    _announce("run-to-run determinism")
    g = torch.Generator().manual_seed(9)
    q, k, v = (torch.randn(2, 4, 1000, 128, generator=g).half().cuda() for _ in range(3))
    a = _run(q, k, v, qk_quant_gran="per_warp", smooth_v=True)
    for _ in range(3):
        assert torch.equal(a, _run(q, k, v, qk_quant_gran="per_warp", smooth_v=True))


# ------------------------------------------------------------------ degenerate inputs
def test_all_zero_k_gives_uniform_attention():
    """K = 0 makes every score 0: the output is the mean of V over visible keys."""
    _announce("all-zero K")
    g = torch.Generator().manual_seed(10)
    q = torch.randn(1, 2, 150, 64, generator=g).half().cuda()
    k = torch.zeros(1, 2, 150, 64).half().cuda()
    v = torch.randn(1, 2, 150, 64, generator=g).half().cuda()
    out = _run(q, k, v, v_dtype="fp16").float().cpu()
    ref = v.float().cpu().mean(dim=2, keepdim=True).expand_as(out)
    assert torch.max(torch.abs(out - ref)) < 2e-3
    outc = _run(q, k, v, v_dtype="fp16", is_causal=True).float().cpu()
    refc = v.float().cpu().cumsum(dim=2) / torch.arange(1, 151).view(1, 1, 150, 1)
    assert torch.max(torch.abs(outc - refc)) < 2e-3


@pytest.mark.parametrize("d, gran", [(128, "per_warp"), (128, "per_thread"), (64, "per_block"), (64, "per_thread")])
def test_causal_zero_scales_fp8_v(d, gran):
    """Causal FP8-V attention with zero scale factors on the diagonal tiles:
    head 0's keys are all equal, so smooth_k leaves K at zero and every K
    scale is 0; rows 100-299 of Q are zero (Q scale 0).  Every score is then
    0, and masked keys must still get no weight.  Checked against the oracle
    and exact attention; at 128 channels the call that quantizes Q in the
    attention kernel must give the same bits."""
    base = workloads.WORKLOADS["b2h8n4096d128"]
    w = dataclasses.replace(base, B=1, Hq=2, Hkv=2, Nq=700, Nk=700, d=d, gran=gran, causal=True, seed=31)
    _announce(f"causal zero scales: B1 H2 N700 d{d} {gran} V=fp8 seed 31")
    inp = workloads.make_inputs(w)
    k = inp["k"].clone()
    k[:, 0] = k[:, 0, :1]                                   # HND: head 0's keys all equal to its first
    q = inp["q"].clone()
    q[:, :, 100:300] = 0
    inp["k"], inp["q"] = k, q
    c = Case(w, inp).run_gpu(return_lse=True).run_oracle(exact=True)
    c.check_quantized_bitexact()
    c.check_outputs(lse=True)
    if sage.q_fusable(q.cuda(), 1, 2, 2, 700, d, gran, "fp8", True, False, (q.stride(0), q.stride(1), q.stride(2))):
        qc, kc, vc = q.cuda(), k.cuda(), inp["v"].cuda()
        kw = dict(tensor_layout="HND", qk_quant_gran=gran, smooth_k=True, v_dtype="fp8", smooth_v=w.smooth_v)
        ref = sage.sage_attn_fwd(*sage.sage_quant_qkv(qc, kc, vc, **kw), is_causal=True, return_lse=True)
        fused = sage.sage_attn_fwd(*sage.sage_quant_qkv(qc, kc, vc, quantize_q=False, **kw), is_causal=True,
                                   return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(ref[0].view(torch.int16), fused[0].view(torch.int16))
        assert torch.equal(ref[1], fused[1])


def test_single_key_returns_its_value():
    _announce("one key")
    g = torch.Generator().manual_seed(11)
    q = torch.randn(1, 1, 70, 32, generator=g).half().cuda()
    k = torch.randn(1, 1, 1, 32, generator=g).half().cuda()
    v = torch.randn(1, 1, 1, 32, generator=g).half().cuda()
    out = _run(q, k, v, v_dtype="fp16")
    assert torch.equal(out, v.expand(1, 1, 70, 32))


def test_page_shape_examples():
    """The shape/dtype examples the pages print (tests/golden/page_shapes.txt)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.txt")
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        src, shape, layout, causal, dtype, out_shape = [t.strip() for t in line.split("|")]
        shape = tuple(int(x) for x in shape.split(","))
        _announce(f"page example {shape} {layout} causal={causal}")
        g = torch.Generator().manual_seed(42)
        q, k, v = (torch.randn(*shape, generator=g).half().cuda() for _ in range(3))
        out = _run(q, k, v, tensor_layout=layout, is_causal=bool(int(causal)))
        assert tuple(out.shape) == tuple(int(x) for x in out_shape.split(",")), src
        assert out.dtype == torch.float16
        # loose sanity bound from the AMD page's test (mean abs diff vs SDPA around 1e-2)
        ref = torch.nn.functional.scaled_dot_product_attention(q.float(), k.float(), v.float(),
                                                               is_causal=bool(int(causal)))
        assert (out.float() - ref).abs().mean().item() < 1e-2


# ------------------------------------------------------------------ fused quantize call
def _quant_pair(inp, w, fused, v_dtype=None, smooth_v=None):
    dev = "cuda"
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    vd = v_dtype or w.v_dtype
    sv = w.smooth_v if smooth_v is None else smooth_v
    kw = {}
    if w.varlen:
        cu = inp["cu_seqlens"].to(dev)
        ms = inp["max_seqlen"]
        kw = dict(cu_seqlens_k=cu, max_seqlen_k=ms)
        kq = dict(cu_seqlens_q=cu, max_seqlen_q=ms)
    else:
        kw = dict(tensor_layout=w.layout)
        kq = {}
    if fused:
        return sage.sage_quant_qkv(q, k, v, qk_quant_gran=w.gran, smooth_k=w.smooth_k, v_dtype=vd, smooth_v=sv,
                                   **kq, **kw)
    qk = sage.sage_quant_qk(q, k, qk_quant_gran=w.gran, smooth_k=w.smooth_k, **kq, **kw)
    qv = sage.sage_quant_v(v, v_dtype=vd, smooth_v=sv, **kw)
    return qk, qv


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER)
def test_fused_quantize_equals_separate_calls(name):
    """sage_quant_qkv (two launches) writes the same bits as sage_quant_qk +
    sage_quant_v (four launches), on every workload at full size."""
    w = workloads.WORKLOADS[name]
    _announce(f"fused quantize {name}")
    inp = workloads.make_inputs(w)
    a_qk, a_v = _quant_pair(inp, w, fused=False)
    b_qk, b_v = _quant_pair(inp, w, fused=True)
    torch.cuda.synchronize()
    lens = inp["lens"] if w.varlen else None
    a, b = written_quant_outputs(a_qk, a_v, lens), written_quant_outputs(b_qk, b_v, lens)
    for f in a:
        assert (a[f] is None) == (b[f] is None), f
        if a[f] is not None:
            assert torch.equal(a[f], b[f]), f


@pytest.mark.parametrize("v_dtype,smooth_v", [("fp8", True), ("fp16", False), ("fp16", True)])
def test_fused_quantize_equals_separate_calls_v_modes(v_dtype, smooth_v):
    w = dataclasses.replace(workloads.WORKLOADS["gqa_prefill_n8192"], Nq=1000, Nk=1000)
    _announce(f"fused quantize v_dtype={v_dtype} smooth_v={smooth_v} (GQA prefill recipe, N=1000)")
    inp = workloads.make_inputs(w)
    a_qk, a_v = _quant_pair(inp, w, fused=False, v_dtype=v_dtype, smooth_v=smooth_v)
    b_qk, b_v = _quant_pair(inp, w, fused=True, v_dtype=v_dtype, smooth_v=smooth_v)
    torch.cuda.synchronize()
    for x, y in ((a_qk.q8, b_qk.q8), (a_qk.k8, b_qk.k8), (a_qk.k_scale, b_qk.k_scale), (a_v.vt, b_v.vt)):
        assert torch.equal(x, y)
    for x, y in ((a_v.v_scale, b_v.v_scale), (a_v.v_mean, b_v.v_mean)):
        assert (x is None) == (y is None)
        if x is not None:
            assert torch.equal(x, y)
