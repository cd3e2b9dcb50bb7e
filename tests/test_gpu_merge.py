"""GPU parity of the merge of partial attention results (needs an MI355X).

sage_merge_states against the oracle's fp64 merge (oracle.merge_states) on
the same seeded partial outputs and log-sum-exps (workloads.make_merge_inputs),
element by element.  The kernel works in fp32 and rounds once to fp16/bf16,
so each output may differ from the fp64 value by one output ulp plus the
fp32 error of the weights and the S-term sum, bounded here by
1e-5 * max_s |o_s| of the row; the merged log-sum-exp by 1e-5 * (1 + |L|).
Rows whose parts all saw no key must give exactly 0 and -inf.

Also a property at any size: attention over two halves of the keys, each a
quantized forward with return_lse, merged, is within the method's tolerance
of exact attention over all keys (cosine >= 0.999).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import quantized_attention_smooth_amd as sage
from parity_utils import cosine, out_ulp

pytestmark = pytest.mark.gpu

CASES = [
    # S, B, H, N, d, dtype, layout
    (2, 2, 8, 4096, 128, "fp16", "HND"),     # two halves of the 4096-token benchmark shape
    (1, 1, 2, 33, 64, "fp16", "HND"),
    (3, 1, 4, 257, 128, "bf16", "NHD"),
    (5, 2, 3, 100, 72, "fp16", "HND"),       # d not a multiple of 8: one channel per thread
    (4, 1, 2, 65, 8, "bf16", "HND"),
    (2, 1, 1, 1, 1, "fp16", "NHD"),
    (16, 1, 2, 300, 64, "bf16", "NHD"),
    (64, 1, 1, 40, 128, "fp16", "HND"),      # the largest number of parts the call accepts
    (2, 1, 2, 5, 1024, "bf16", "HND"),       # the largest head size the call accepts
]


def _check(got_o, got_l, inp):
    S, B, H, N, d = inp["shape"]
    layout = inp["layout"]
    parts = inp["out_parts"].float().numpy()
    if layout == "NHD":
        parts = parts.transpose(0, 1, 3, 2, 4)
        got_o = got_o.transpose(0, 2, 1, 3)
    parts = parts.reshape(S, B * H * N, d)
    L = inp["lse_parts"].numpy().reshape(S, B * H * N)
    ref_o, ref_l = oracle.merge_states(parts, L)
    got_o = got_o.reshape(B * H * N, d).astype(np.float64)
    got_l = got_l.reshape(-1).astype(np.float64)
    scale = np.abs(parts).max(axis=(0, 2))[:, None]
    tol = out_ulp(ref_o, inp["dtype"]) + 1e-5 * scale
    bad = np.abs(got_o - ref_o) > tol
    assert not bad.any(), (f"{bad.sum()} outputs off; worst |diff| "
                           f"{np.abs(got_o - ref_o).max():.3g} at {np.unravel_index(np.argmax(np.abs(got_o - ref_o)), bad.shape)}")
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty)
    assert np.all(got_o[empty] == 0.0)
    ok = ~empty
    assert np.all(np.abs(got_l[ok] - ref_l[ok]) <= 1e-5 * (1 + np.abs(ref_l[ok])))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "S{}_B{}_H{}_N{}_d{}_{}_{}".format(*c))
def test_merge_matches_oracle(case):
    S, B, H, N, d, dtype, layout = case
    print(f"[gpu-case] merge S={S} B={B} H={H} N={N} d={d} {dtype} {layout} seed 21", flush=True)
    inp = workloads.make_merge_inputs(21, S, B, H, N, d, dtype, layout)
    dev = torch.device("cuda:0")
    o, l = sage.sage_merge_states(inp["out_parts"].to(dev), inp["lse_parts"].to(dev), tensor_layout=layout)
    torch.cuda.synchronize()
    _check(o.float().cpu().numpy(), l.cpu().numpy(), inp)


def test_merge_into_strided_output():
    print("[gpu-case] merge into a strided view, S=3 B=1 H=2 N=50 d=64 fp16 HND seed 22", flush=True)
    inp = workloads.make_merge_inputs(22, 3, 1, 2, 50, 64, "fp16", "HND")
    dev = torch.device("cuda:0")
    big = torch.full((1, 2, 50, 100), 7.0, dtype=torch.float16, device=dev)
    view = big[..., 3:67]                                   # rows 200 bytes apart, 6-byte offset
    o, l = sage.sage_merge_states(inp["out_parts"].to(dev), inp["lse_parts"].to(dev), out=view)
    torch.cuda.synchronize()
    _check(view.float().cpu().numpy(), l.cpu().numpy(), inp)
    rest = torch.cat([big[..., :3], big[..., 67:]], dim=-1)
    assert bool((rest == 7.0).all())                        # nothing written outside the view


def test_split_key_attention_merges_to_full_attention():
    w = workloads.WORKLOADS["b2h8n4096d128"]
    print("[gpu-case] split-key attention + merge: B1 H4 N1024 d128 fp16 per_warp FP8 V, seed 2", flush=True)
    inp = workloads.make_inputs(w, {"B": 1, "Hq": 4, "Hkv": 4, "Nq": 1024, "Nk": 1024})
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    outs, lses = [], []
    for a, b in ((0, 384), (384, 1024)):
        o, l = sage.sageattn(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), return_lse=True,
                             qk_quant_gran="per_warp")
        outs.append(o); lses.append(l)
    mo, ml = sage.sage_merge_states(torch.stack(outs), torch.stack(lses).contiguous())
    torch.cuda.synchronize()
    ex = oracle.exact_forward(*(inp[x].float().numpy() for x in ("q", "k", "v")))
    ref_o, ref_l = ex["out"][0], ex["lse"][0]
    got_o = mo.float().cpu().numpy()[0]
    assert cosine(got_o, ref_o) >= 0.999
    assert np.abs(ml.cpu().numpy()[0] - ref_l).max() < 0.05
