"""Host-side contract of bench.py (no GPU): it refuses more than one GPU, its
TOPS numerators are the operation counts of the workloads, and the sequence
sweep keeps the same number of query tokens at every length."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name, ops", [
    ("b2h8n4096d128", 2.0 ** 37),                      # 4 * 2 * 8 * 4096^2 * 128
    ("gqa_prefill_n8192", 2.0 ** 40 / 2),              # 4 * 32 * 8192^2 * 128, causal
    ("video_dit_n17550", 4.0 * 48 * 17550 ** 2 * 64),  # 3.785e12
    ("tiny", 4.0 * 2 * 256 ** 2 * 64),
])
def test_attention_ops(name, ops):
    assert workloads.attention_ops(workloads.WORKLOADS[name]) == ops


def test_varlen_ops_sum_per_sequence():
    w = workloads.WORKLOADS["varlen16_h16"]
    lens = [100, 4096, 1]
    expect = 4.0 * w.Hq * w.d * sum(n * n for n in lens)
    assert workloads.attention_ops(w, lens=lens) == (expect / 2 if w.causal else expect)


def test_sweep_keeps_token_count():
    assert bench.SWEEP_N[0] == 1024 and bench.SWEEP_N[-1] == 32768
    for n in bench.SWEEP_N:
        assert bench.SWEEP_TOKENS % n == 0


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.kernel_source_hash()


def test_peaks():
    assert bench.PEAK_TOPS["fp8"] == 5000.0
    assert abs(bench.PEAK_TOPS["fp16"] - 10000.0 / 3.0) < 1e-9
