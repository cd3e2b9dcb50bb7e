"""Host-side logic of the Python binding that needs no GPU: argument checks
that raise before any library call, and the split-KV range-count plan."""
import numpy as np
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


def test_attention_takes_q_in_its_input_precision_only_where_groups_fit_a_tile():
    """The C ABI's rule (pure host code): FP8 V, head_dim a multiple of 8 above 64, and
    with packed query heads (grouped heads, non-causal, dense, Nq <= 128)
    whole quantization groups per head."""
    L = sage.load_library()
    P_THREAD, P_WARP, P_BLOCK = 2, 1, 0
    FP8, FP16 = 0, 1

    def ok(B, Hq, Hkv, Nq, d, gran, vd=FP8, causal=0, varlen=0):
        return L.sage_attn_q_fusable(B, Hq, Hkv, Nq, d, gran, vd, causal, varlen) == 1

    assert (sage.api._GRAN["per_thread"], sage.api._GRAN["per_warp"], sage.api._GRAN["per_block"]) == \
        (P_THREAD, P_WARP, P_BLOCK)
    assert ok(2, 8, 8, 4096, 128, P_WARP)
    assert not ok(2, 8, 8, 4096, 128, P_WARP, vd=FP16)         # the FP16-V kernel reads INT8 Q
    assert not ok(2, 8, 8, 4096, 100, P_WARP)                   # 8-channel slices
    assert ok(2, 8, 8, 4096, 96, P_BLOCK)
    assert not ok(2, 8, 8, 4096, 64, P_THREAD)                  # the 64-channel kernel reads INT8 Q
    assert ok(4, 32, 8, 17, 128, P_THREAD)                      # packed rows: one row per group
    assert not ok(4, 32, 8, 40, 128, P_WARP)                    # packed rows: a group would straddle heads
    assert ok(4, 32, 8, 64, 128, P_WARP)
    assert not ok(4, 32, 8, 64, 128, P_BLOCK)
    assert ok(4, 32, 8, 128, 128, P_BLOCK)
    assert ok(4, 32, 8, 40, 128, P_WARP, causal=1)              # causal calls are not packed
    assert ok(4, 32, 8, 40, 128, P_WARP, varlen=1)              # nor varlen ones
    assert ok(4, 32, 8, 200, 128, P_WARP)                       # more than 128 queries: not packed
    assert not ok(1, 6, 4, 64, 128, P_WARP)                     # Hq not a multiple of Hkv
    assert not ok(1, 8, 8, 64, 128, 7)                          # unknown granularity


def test_sageattn_splits_automatically_only_when_compute_units_idle():
    assert sage.auto_kv_splits(2, 8, 8, 4096, 4096, False) == 1            # 256 row tiles fill the GPU
    n = sage.auto_kv_splits(4, 32, 8, 16, 32768, False)                      # decode: 32 packed row tiles
    assert n == sage.splitkv_plan(4, 32, 16, 32768, Hkv=8) and n >= 2
    assert sage.auto_kv_splits(4, 32, 8, 16, 32768, True) == 1              # causal calls run one pass
    assert sage.auto_kv_splits(4, 32, 8, 16, 32768, False, None) == 1       # None: one pass
    assert sage.auto_kv_splits(4, 32, 8, 16, 32768, False, 3) == 3
    # ranges of at least 1024 keys: a small call stays one pass
    assert sage.splitkv_plan(1, 2, 640, 640) >= 2 and sage.auto_kv_splits(1, 2, 2, 640, 640, False) == 1
    assert sage.auto_kv_splits(2, 8, 8, 8, 5000, False) == 4              # 16 by the plan, 4 by the key count
    with pytest.raises(NotImplementedError):
        sage.auto_kv_splits(1, 1, 1, 1, 1, True, 2)
    with pytest.raises(ValueError):
        sage.auto_kv_splits(1, 1, 1, 1, 1, False, 0)


def test_sageattn_refuses_cpu_tensors():
    q = torch.zeros(1, 2, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):                     # CPU tensors are refused first
        sage.sageattn(q, q, q, kv_splits=2)


# ---------------------------------------------------------------- caller-supplied outputs
def _cpu_quantized(B=1, Hq=2, Hkv=2, N=130, d=64):
    """Quantized-operand holders with CPU tensors: the binding's output checks
    run before any call into the library, so no GPU is needed."""
    import torch
    from quantized_attention_smooth_amd.api import QuantQK, QuantV
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt)
    qk = QuantQK(z(B, Hq, 256, 64, dt=torch.int8), z(B, Hq, 256), z(B, Hkv, 256, 64, dt=torch.int8), z(B, Hkv, 16),
                 z(B, Hkv, 64), "per_thread", B, Hq, Hkv, N, N, d, torch.float16)
    qv = QuantV(z(B, Hkv, 64, 256, dt=torch.uint8), z(B, Hkv, 64), None, "fp8")
    return qk, qv


@pytest.mark.parametrize("bad", ["shape", "dtype", "layout"])
def test_attn_fwd_rejects_wrong_out(bad):
    import torch
    import quantized_attention_smooth_amd as sage
    qk, qv = _cpu_quantized()
    shape, dt = (1, 2, 130, 64), torch.float16
    if bad == "shape":
        shape = (1, 2, 129, 64)
    if bad == "dtype":
        dt = torch.float32
    out = torch.empty(shape, dtype=dt)
    layout = "NHD" if bad == "layout" else "HND"           # HND-shaped out for an NHD call
    with pytest.raises(ValueError):
        sage.sage_attn_fwd(qk, qv, out=out, tensor_layout=layout)
    with pytest.raises(ValueError):
        sage.sage_attn_fwd_splitkv(qk, qv, out=out, tensor_layout=layout, n_splits=2)


def test_attn_varlen_and_merge_reject_wrong_out():
    import torch
    import quantized_attention_smooth_amd as sage
    qk, qv = _cpu_quantized(B=3)
    cu = torch.tensor([0, 50, 90, 130], dtype=torch.int32)
    with pytest.raises(ValueError):
        sage.sage_attn_varlen_fwd(qk, qv, cu, cu, 130, out=torch.empty((129, 2, 64), dtype=torch.float16))
    parts = torch.zeros((2, 1, 2, 10, 64), dtype=torch.float16)
    lse = torch.zeros((2, 1, 2, 10), dtype=torch.float32)
    for out in (torch.empty((1, 2, 10, 32), dtype=torch.float16), torch.empty((1, 2, 10, 64), dtype=torch.bfloat16)):
        with pytest.raises(ValueError):
            sage.sage_merge_states(parts, lse, out=out)


# ---------------------------------------------------------------- SDPA call convention
@pytest.mark.parametrize("kw", [dict(attn_mask=torch.zeros(1)), dict(dropout_p=0.1)])
def test_sdpa_convention_unsupported_raises_not_implemented(kw):
    """A mask or dropout is refused with NotImplementedError (before any
    library call), which an SDPA caller can catch to fall back."""
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    with pytest.raises(NotImplementedError):
        sage.sageattn(q, q, q, **kw)


def test_sdpa_positional_mask_is_recognised():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    with pytest.raises(NotImplementedError):
        sage.sageattn(q, q, q, torch.zeros(8, 8))          # SDPA order: attn_mask fourth
    with pytest.raises(NotImplementedError):
        sage.sageattn(q, q, q, None, 0.5)                  # dropout_p fifth
    with pytest.raises(ValueError):                        # supported call, but CPU tensors
        sage.sageattn(q, q, q, None, 0.0, True, 0.1)


# ---------------------------------------------------------------- bf16 mean exactness condition
def test_bf16_sum_exactness_condition():
    from parity_utils import bf16_sum_exact_in_fp64 as ok
    assert ok(np.array([1.0, 2.0 ** -45]))                 # u = 2^-52: 1 < 2^53 u = 2
    assert not ok(np.array([1.0, 2.0 ** -46]))             # u = 2^-53: 1 + 2^-46 >= 2^53 u = 1
    assert ok(np.zeros(5)) and ok(np.array([0.0, -3.0]))
    assert ok(np.array([2.0 ** -133, 2.0 ** -120]))        # subnormal ulp 2^-133
    # the condition is what it claims: fp64 sums of such columns are exact in any order
    import math
    rng = np.random.default_rng(5)
    for _ in range(20):
        e = rng.integers(-20, 18, 64)
        x = rng.choice([-1.0, 1.0], 64) * (1 + rng.integers(0, 128, 64) / 128) * np.exp2(e)
        if ok(x):
            exact = math.fsum(x.tolist())
            for order in (x, x[::-1], rng.permutation(x)):
                s = 0.0
                for v in order:
                    s += float(v)
                assert s == exact
