"""Build libsage.so (gfx950 code objects + the C ABI) in-tree with hipcc.

    python -m quantized_attention_smooth_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU
instructions disabled, and linked into quantized_attention_smooth_amd/libsage.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsage.so")
SOURCES = ["quant.hip", "attn.hip", "merge.hip", "sage_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-result",
]


# The attention kernel keeps MFMA results in VGPRs (its softmax reads the score
# accumulators directly); its output accumulators are placed in AGPRs by the
# kernel's own inline-assembly MFMAs.
EXTRA = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed for {src}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libsage.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
