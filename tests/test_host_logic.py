"""Host-side logic of the Python binding that needs no GPU: argument checks
that raise before any library call, and the split-KV range-count plan."""
import pytest
import torch

import oracle
import quantized_attention_smooth_amd as sage


def _parts(S=2, B=1, H=2, N=4, d=8, dtype=torch.float16):
    return torch.zeros(S, B, H, N, d, dtype=dtype), torch.zeros(S, B, H, N, dtype=torch.float32)


@pytest.mark.parametrize("case", ["4-D parts", "fp32 parts", "lse shape", "lse dtype", "lse not contiguous",
                                  "layout", "channel stride"])
def test_merge_rejects_before_any_call(case):
    o, l = _parts()
    kw = {}
    if case == "4-D parts":
        o = o[0]
    elif case == "fp32 parts":
        o = o.float()
    elif case == "lse shape":
        l = l[:, :, :, :3]
    elif case == "lse dtype":
        l = l.double()
    elif case == "lse not contiguous":
        l = torch.zeros(2, 1, 4, 2).permute(0, 1, 3, 2)
    elif case == "layout":
        kw["tensor_layout"] = "BHSD"
    elif case == "channel stride":
        o = torch.zeros(2, 1, 2, 8, 4, dtype=torch.float16).transpose(3, 4)
    with pytest.raises(ValueError):
        sage.sage_merge_states(o, l, **kw)


def test_splitkv_plan():
    # explicit request is passed through
    assert sage.splitkv_plan(1, 8, 16, 4096, n_splits=7) == 7
    # as many ranges as fit one round of 256 workgroups, ranges of at least 256 keys, at most 64
    assert sage.splitkv_plan(1, 8, 16, 32768, Hkv=8) == 32
    assert sage.splitkv_plan(1, 8, 16, 1024, Hkv=8) == 4
    assert sage.splitkv_plan(4, 32, 2048, 32768, Hkv=32) == 1
    assert sage.splitkv_plan(1, 1, 16, 1 << 20) == 64
    assert sage.splitkv_plan(1, 3, 16, 1 << 20) == 64          # 3 tiles x 64 ranges = 192 workgroups
    assert sage.splitkv_plan(1, 5, 16, 1 << 20) == 51          # 5 x 51 = 255 <= 256
    # packed GQA rows: the 4 query heads of a K/V head share one row tile
    assert sage.splitkv_plan(4, 32, 16, 32768, Hkv=8) == 8
    assert sage.splitkv_plan(4, 32, 200, 32768, Hkv=8) == 2       # 200 > 128 queries: not packed
    for B, Hq, Hkv, Nq, Nk in [(1, 1, 1, 1, 1), (2, 64, 8, 33, 100000), (16, 16, 16, 4096, 4096)]:
        n = sage.splitkv_plan(B, Hq, Nq, Nk, Hkv=Hkv)
        assert 1 <= n <= 64
        assert n == 1 or n * (B * Hkv if Hq > Hkv and Nq <= 128 else B * Hq) <= 256
        assert len(oracle.splitkv_ranges(Nk, n)) <= n


def test_sageattn_refuses_cpu_tensors():
    q = torch.zeros(1, 2, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):                     # CPU tensors are refused first
        sage.sageattn(q, q, q, kv_splits=2)
