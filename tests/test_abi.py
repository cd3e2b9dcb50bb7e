"""Host-side checks of the C ABI (no GPU needed).

* libsage.so loads and exports every function include/sage.h declares;
* the Python ctypes mirrors have the C structs' exact layout (compiled here
  with gcc against include/sage.h);
* every argument check fails with SAGE_EINVAL and a message before any HIP
  call: each case below breaks exactly one rule of an otherwise valid call.
"""
import ctypes
import os
import re
import subprocess

import pytest

from quantized_attention_smooth_amd import _abi as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")


@pytest.fixture(scope="module")
def lib():
    return A.load()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(sage_[a-z_0-9]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(A.EXPORTS), declared
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(sage_\w+)", out))
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    assert lib.sage_version() == 1


def test_struct_layouts_match_c(tmp_path):
    structs = {
        "sage_quant_qk_params": A.QuantQKParams,
        "sage_quant_v_params": A.QuantVParams,
        "sage_attn_params": A.AttnParams,
        "sage_merge_params": A.MergeParams,
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "sage.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append('printf("sage_attn_varlen_params size %zu\\n", sizeof(sage_attn_varlen_params));')
    for f in ("cu_seqlens_q", "cu_seqlens_k", "total_q"):
        lines.append(f'printf("sage_attn_varlen_params {f} %zu\\n", offsetof(sage_attn_varlen_params, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = {}
    for line in subprocess.check_output([str(exe)], text=True).splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
    assert got[("sage_attn_varlen_params", "size")] == ctypes.sizeof(A.AttnVarlenParams)
    for f in ("cu_seqlens_q", "cu_seqlens_k", "total_q"):
        assert got[("sage_attn_varlen_params", f)] == getattr(A.AttnVarlenParams, f).offset


# fake, well-aligned device addresses: validation never dereferences them
FAKE = 0x7F0000000000


def _qk_valid():
    p = A.QuantQKParams()
    p.struct_size = ctypes.sizeof(p)
    p.q, p.k, p.dtype = FAKE, FAKE + 0x100000, A.SAGE_F16
    p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d = 1, 4, 2, 100, 120, 64
    p.q_stride_b, p.q_stride_h, p.q_stride_n = 4 * 100 * 64, 100 * 64, 64
    p.k_stride_b, p.k_stride_h, p.k_stride_n = 2 * 120 * 64, 120 * 64, 64
    p.gran, p.smooth_k = A.SAGE_PER_THREAD, 1
    p.q8, p.q_scale, p.k8, p.k_scale, p.k_mean = (FAKE + i * 0x100000 for i in range(2, 7))
    p.workspace = FAKE + 0x800000
    p.workspace_bytes = 1 << 20
    return p


QK_BREAKS = {
    "struct_size": lambda p: setattr(p, "struct_size", 8),
    "dtype": lambda p: setattr(p, "dtype", 7),
    "head_dim 129": lambda p: setattr(p, "d", 129),
    "head_dim 0": lambda p: setattr(p, "d", 0),
    "Hq not multiple of Hkv": lambda p: setattr(p, "Hkv", 3),
    "Nk = 0": lambda p: setattr(p, "Nk", 0),
    "B = 0": lambda p: setattr(p, "B", 0),
    "gran": lambda p: setattr(p, "gran", 5),
    "null q": lambda p: setattr(p, "q", None),
    "null k8": lambda p: setattr(p, "k8", None),
    "null k_mean with smooth_k": lambda p: setattr(p, "k_mean", None),
    "q8 misaligned": lambda p: setattr(p, "q8", FAKE + 0x200008),
    "scale misaligned": lambda p: setattr(p, "k_scale", FAKE + 0x500002),
    "only one cu_seqlens": lambda p: setattr(p, "cu_seqlens_q", FAKE + 0x900000),
    "zero token stride": lambda p: setattr(p, "q_stride_n", 0),
    "workspace too small": lambda p: setattr(p, "workspace_bytes", 16),
    "workspace null": lambda p: setattr(p, "workspace", None),
}


@pytest.mark.parametrize("case", list(QK_BREAKS))
def test_quant_qk_rejects(lib, case):
    p = _qk_valid()
    QK_BREAKS[case](p)
    assert lib.sage_quant_qk(ctypes.byref(p), None) == A.SAGE_EINVAL
    assert len(lib.sage_last_error()) > 0


def _v_valid():
    p = A.QuantVParams()
    p.struct_size = ctypes.sizeof(p)
    p.v, p.dtype = FAKE, A.SAGE_BF16
    p.B, p.Hkv, p.Nk, p.d = 2, 2, 300, 128
    p.v_stride_b, p.v_stride_h, p.v_stride_n = 300 * 2 * 128, 128, 2 * 128
    p.v_dtype, p.smooth_v = A.SAGE_V_FP8, 1
    p.vt, p.v_scale, p.v_mean = FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000
    p.workspace, p.workspace_bytes = FAKE + 0x400000, 1 << 22
    return p


V_BREAKS = {
    "v_dtype": lambda p: setattr(p, "v_dtype", 9),
    "fp8 without v_scale": lambda p: setattr(p, "v_scale", None),
    "smooth_v without v_mean": lambda p: setattr(p, "v_mean", None),
    "vt misaligned": lambda p: setattr(p, "vt", FAKE + 0x100004),
    "head_dim 200": lambda p: setattr(p, "d", 200),
    "workspace too small": lambda p: setattr(p, "workspace_bytes", 1000),
    "negative stride": lambda p: setattr(p, "v_stride_h", -128),
}


@pytest.mark.parametrize("case", list(V_BREAKS))
def test_quant_v_rejects(lib, case):
    p = _v_valid()
    V_BREAKS[case](p)
    assert lib.sage_quant_v(ctypes.byref(p), None) == A.SAGE_EINVAL
    assert len(lib.sage_last_error()) > 0


def _attn_valid():
    p = A.AttnParams()
    p.struct_size = ctypes.sizeof(p)
    p.q8, p.q_scale, p.k8, p.k_scale, p.k_mean = (FAKE + i * 0x100000 for i in range(5))
    p.vt, p.v_scale, p.v_mean = FAKE + 0x600000, FAKE + 0x700000, None
    p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d = 2, 8, 8, 256, 256, 128
    p.gran, p.v_dtype, p.pv_accum, p.is_causal, p.sm_scale = A.SAGE_PER_WARP, A.SAGE_V_FP8, A.SAGE_ACC_FP16_FP32, 0, 0.0
    p.in_dtype, p.out, p.out_dtype = A.SAGE_F16, FAKE + 0x900000, A.SAGE_F16
    p.o_stride_b, p.o_stride_h, p.o_stride_n = 8 * 256 * 128, 256 * 128, 128
    return p


ATTN_BREAKS = {
    "struct_size": lambda p: setattr(p, "struct_size", 4),
    "head_dim 129": lambda p: setattr(p, "d", 129),
    "GQA mismatch": lambda p: setattr(p, "Hkv", 3),
    "Nq = 0": lambda p: setattr(p, "Nq", 0),
    "pv_accum": lambda p: setattr(p, "pv_accum", 11),
    "v_dtype": lambda p: setattr(p, "v_dtype", 2),
    "out dtype": lambda p: setattr(p, "out_dtype", 3),
    "null out": lambda p: setattr(p, "out", None),
    "null vt": lambda p: setattr(p, "vt", None),
    "fp8 without v_scale": lambda p: setattr(p, "v_scale", None),
    "k8 misaligned": lambda p: setattr(p, "k8", FAKE + 0x200001),
    "lse misaligned": lambda p: setattr(p, "lse", FAKE + 0xA00002),
    "sm_scale nan": lambda p: setattr(p, "sm_scale", float("nan")),
    "sm_scale inf": lambda p: setattr(p, "sm_scale", float("inf")),
    "zero out stride": lambda p: setattr(p, "o_stride_n", 0),
}


@pytest.mark.parametrize("case", list(ATTN_BREAKS))
def test_attn_rejects(lib, case):
    p = _attn_valid()
    ATTN_BREAKS[case](p)
    assert lib.sage_attn_fwd(ctypes.byref(p), None) == A.SAGE_EINVAL
    assert len(lib.sage_last_error()) > 0


def test_attn_varlen_rejects(lib):
    vp = A.AttnVarlenParams()
    vp.base = _attn_valid()
    vp.base.struct_size = ctypes.sizeof(A.AttnParams)          # too small for the varlen struct
    vp.cu_seqlens_q, vp.cu_seqlens_k, vp.total_q = FAKE + 0xB00000, FAKE + 0xC00000, 500
    assert lib.sage_attn_varlen_fwd(ctypes.byref(vp), None) == A.SAGE_EINVAL
    vp.base.struct_size = ctypes.sizeof(A.AttnVarlenParams)
    vp.cu_seqlens_k = None
    assert lib.sage_attn_varlen_fwd(ctypes.byref(vp), None) == A.SAGE_EINVAL
    vp.cu_seqlens_k = FAKE + 0xC00002
    assert lib.sage_attn_varlen_fwd(ctypes.byref(vp), None) == A.SAGE_EINVAL
    assert lib.sage_attn_varlen_fwd(None, None) == A.SAGE_EINVAL


def test_debug_scores_rejects(lib):
    p = _attn_valid()
    assert lib.sage_debug_qk_scores(ctypes.byref(p), 2, FAKE, None) == A.SAGE_EINVAL
    assert lib.sage_debug_qk_scores(ctypes.byref(p), 0, None, None) == A.SAGE_EINVAL


def test_workspace_size(lib):
    assert lib.sage_quant_workspace_size(0, 1, 1, 64) == 0
    assert lib.sage_quant_workspace_size(1, 1, 1, 129) == 0
    # 8-byte sums + fp32 min/max per (b, h, chunk, channel); about 256 chunks over all heads, 8 to 32 per head,
    # each a multiple of 256 tokens
    n = lib.sage_quant_workspace_size(2, 8, 4096, 128)
    cells = 2 * 8 * 16 * 128
    assert n >= cells * 16
    assert lib.sage_quant_workspace_size(1, 8, 8192, 128) >= 8 * 32 * 128 * 16
    assert lib.sage_quant_workspace_size(1, 48, 17550, 64) >= 48 * 8 * 64 * 16
    assert lib.sage_quant_workspace_size(1, 1, 257, 64) > lib.sage_quant_workspace_size(1, 1, 256, 64)


def _qkv_valid():
    """A matching pair for the fused call: K and V agree and use distinct workspaces."""
    pk = _qk_valid()
    pv = _v_valid()
    pv.dtype, pv.B, pv.Hkv, pv.Nk, pv.d = pk.dtype, pk.B, pk.Hkv, pk.Nk, pk.d
    pv.v_stride_b, pv.v_stride_h, pv.v_stride_n = pk.k_stride_b, pk.k_stride_h, pk.k_stride_n
    pv.workspace, pv.workspace_bytes = FAKE + 0x2000000, 1 << 20
    return pk, pv


QKV_BREAKS = {
    "dtype differs": lambda pk, pv: setattr(pv, "dtype", A.SAGE_BF16),
    "Nk differs": lambda pk, pv: setattr(pv, "Nk", pk.Nk + 1),
    "Hkv differs": lambda pk, pv: setattr(pv, "Hkv", 1),
    "head_dim differs": lambda pk, pv: setattr(pv, "d", 32),
    "cu_seqlens_k differs": lambda pk, pv: (setattr(pk, "cu_seqlens_q", FAKE + 0x3000000),
                                            setattr(pk, "cu_seqlens_k", FAKE + 0x3100000)),
    "workspaces overlap": lambda pk, pv: setattr(pv, "workspace", pk.workspace + 256),
    "K params invalid": lambda pk, pv: setattr(pk, "gran", 7),
    "V params invalid": lambda pk, pv: setattr(pv, "v_dtype", 9),
}


@pytest.mark.parametrize("case", sorted(QKV_BREAKS))
def test_quant_qkv_rejects(lib, case):
    pk, pv = _qkv_valid()
    QKV_BREAKS[case](pk, pv)
    assert lib.sage_quant_qkv(ctypes.byref(pk), ctypes.byref(pv), None) == A.SAGE_EINVAL
    assert len(lib.sage_last_error()) > 0


def test_quant_qkv_null_params(lib):
    pk, pv = _qkv_valid()
    assert lib.sage_quant_qkv(None, ctypes.byref(pv), None) == A.SAGE_EINVAL
    assert lib.sage_quant_qkv(ctypes.byref(pk), None, None) == A.SAGE_EINVAL


def _merge_valid():
    p = A.MergeParams()
    p.struct_size = ctypes.sizeof(p)
    p.n_parts, p.dtype, p.B, p.H, p.N, p.d = 2, A.SAGE_F16, 2, 4, 100, 128
    p.parts = FAKE
    p.ps_s, p.ps_b, p.ps_h, p.ps_n = 2 * 4 * 100 * 128, 4 * 100 * 128, 100 * 128, 128
    p.lse_parts, p.out, p.lse = FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000
    p.o_stride_b, p.o_stride_h, p.o_stride_n = 4 * 100 * 128, 100 * 128, 128
    return p


MERGE_BREAKS = {
    "struct_size": lambda p: setattr(p, "struct_size", 8),
    "no parts": lambda p: setattr(p, "n_parts", 0),
    "65 parts": lambda p: setattr(p, "n_parts", 65),
    "d = 0": lambda p: setattr(p, "d", 0),
    "d = 1025": lambda p: setattr(p, "d", 1025),
    "N = 0": lambda p: setattr(p, "N", 0),
    "dtype": lambda p: setattr(p, "dtype", 4),
    "null parts": lambda p: setattr(p, "parts", None),
    "null lse_parts": lambda p: setattr(p, "lse_parts", None),
    "null out": lambda p: setattr(p, "out", None),
    "parts misaligned": lambda p: setattr(p, "parts", FAKE + 1),
    "lse_parts misaligned": lambda p: setattr(p, "lse_parts", FAKE + 0x1000002),
    "lse misaligned": lambda p: setattr(p, "lse", FAKE + 0x3000001),
}


@pytest.mark.parametrize("case", sorted(MERGE_BREAKS))
def test_merge_rejects(lib, case):
    p = _merge_valid()
    MERGE_BREAKS[case](p)
    assert lib.sage_merge_states(ctypes.byref(p), None) == A.SAGE_EINVAL
    assert len(lib.sage_last_error()) > 0


def test_merge_null_params(lib):
    assert lib.sage_merge_states(None, None) == A.SAGE_EINVAL


SPLIT_BREAKS = {
    "n_splits 0": (lambda p: None, 0, 1 << 24, 0, A.SAGE_EINVAL),
    "n_splits 65": (lambda p: None, 65, 1 << 24, 0, A.SAGE_EINVAL),
    "causal": (lambda p: setattr(p, "is_causal", 1), 4, 1 << 24, 0, A.SAGE_EUNSUPPORTED),
    "workspace too small": (lambda p: None, 4, 4096, 0, A.SAGE_EINVAL),
    "workspace misaligned": (lambda p: None, 4, 1 << 24, 128, A.SAGE_EINVAL),
    "head_dim 129": (lambda p: setattr(p, "d", 129), 4, 1 << 24, 0, A.SAGE_EINVAL),
}


@pytest.mark.parametrize("case", sorted(SPLIT_BREAKS))
def test_splitkv_rejects(lib, case):
    brk, ns, nbytes, off, code = SPLIT_BREAKS[case]
    p = _attn_valid()
    brk(p)
    assert lib.sage_attn_fwd_splitkv(ctypes.byref(p), ns, FAKE + 0x4000000 + off, nbytes, None) == code
    assert len(lib.sage_last_error()) > 0


def test_splitkv_workspace_size(lib):
    assert lib.sage_attn_splitkv_workspace_size(1, 8, 4, 4133, 128, 0) == 0
    assert lib.sage_attn_splitkv_workspace_size(1, 8, 4, 4133, 129, 5) == 0
    # 5 requested ranges of 4133 keys: ranges of 896 keys, 5 of them; fp32
    # partial outputs and LSEs, each region rounded up to 256 bytes
    rows = 5 * 1 * 8 * 4
    want = -(-(rows * 128 * 4) // 256) * 256 + -(-(rows * 4) // 256) * 256
    assert lib.sage_attn_splitkv_workspace_size(1, 8, 4, 4133, 128, 5) == want
    # 7 requested ranges of 1000 keys: ranges of 256 keys, only 4 of them
    rows = 4 * 2 * 3 * 10
    want = -(-(rows * 64 * 4) // 256) * 256 + -(-(rows * 4) // 256) * 256
    assert lib.sage_attn_splitkv_workspace_size(2, 3, 10, 1000, 64, 7) == want


# ---------------------------------------------------------------- the no-alloc quantize call (host checks)
def _pair_valid(B=2, Hkv=2, Nk=300, d=128):
    qk, v = _qk_valid(), _v_valid()
    qk.dtype = v.dtype = A.SAGE_BF16
    qk.B = v.B = B
    qk.Hkv = v.Hkv = Hkv
    qk.Hq = 2 * Hkv
    qk.Nk = v.Nk = Nk
    qk.d = v.d = d
    qk.workspace, qk.workspace_bytes = None, 0           # ignored by the no-alloc call
    v.workspace, v.workspace_bytes = None, 0
    return qk, v


def test_noalloc_scratch_size(lib):
    for B, H, N, d in ((1, 2, 300, 64), (2, 8, 4096, 128), (1, 48, 17550, 64), (4, 8, 32768, 128)):
        assert lib.sage_quant_qkv_noalloc_scratch_size(B, H, N, d) == 2 * lib.sage_quant_workspace_size(B, H, N, d)
    assert lib.sage_quant_qkv_noalloc_scratch_size(0, 2, 300, 64) == 0
    assert lib.sage_quant_qkv_noalloc_scratch_size(1, 2, 300, 129) == 0
    # the workloads of the benchmark fit the static array
    assert lib.sage_quant_qkv_noalloc_scratch_size(1, 48, 17550, 64) <= A.SAGE_QUANT_SCRATCH_BYTES


def test_noalloc_rejects_too_large_before_any_hip_call(lib):
    """Beyond the static array the call fails with SAGE_EINVAL on the host
    (no GPU is touched: this runs without one)."""
    qk, v = _pair_valid(B=64, Hkv=32, Nk=100000, d=128)
    assert lib.sage_quant_qkv_noalloc_scratch_size(64, 32, 100000, 128) > A.SAGE_QUANT_SCRATCH_BYTES
    assert lib.sage_quant_qkv_noalloc(ctypes.byref(qk), ctypes.byref(v), None) == A.SAGE_EINVAL
    assert b"too large for the no-alloc call" in lib.sage_last_error()


@pytest.mark.parametrize("case", ["dtype", "head_dim 129", "Hq not multiple of Hkv", "null k8", "q8 misaligned"])
def test_noalloc_rejects_invalid(lib, case):
    qk, v = _pair_valid()
    QK_BREAKS[case](qk)
    assert lib.sage_quant_qkv_noalloc(ctypes.byref(qk), ctypes.byref(v), None) == A.SAGE_EINVAL
    qk, v = _pair_valid()
    v.Nk = 301                                           # K and V disagree
    assert lib.sage_quant_qkv_noalloc(ctypes.byref(qk), ctypes.byref(v), None) == A.SAGE_EINVAL
