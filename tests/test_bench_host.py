"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the
kernel-code hash that gates the counter traffic, the target-row arithmetic,
and the CPU baseline's claim that the threaded oracle run gives the same
bytes as the single-threaded one.
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_code_hash_ignores_comments_and_layout(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* header */\nint f(int x)   {   return x + 1; }\n// trailing\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_code_hash(str(a)) == bench.kernel_code_hash(str(b))
    assert bench.kernel_code_hash(str(a)) != bench.kernel_code_hash(str(c))


def test_counter_traffic_follows_the_kernel_hash(monkeypatch):
    text = open(bench.PROFILE_PMC).read()
    recorded = text.split("kernel_code_sha256_16:")[1].split()[0]
    monkeypatch.setattr(bench, "kernel_code_hash", lambda path=bench.KERNEL_SRC: recorded)
    t = bench.counter_traffic()
    assert t is not None
    # Counter bytes can only exceed the algorithmic bytes (re-reads, partial
    # lines), and not by much for a streaming kernel.
    alg = bench.TOKENS * bench.INSERT_BYTES_PER_TOKEN
    assert alg <= t <= 1.2 * alg
    monkeypatch.setattr(bench, "kernel_code_hash", lambda path=bench.KERNEL_SRC: "0" * 16)
    assert bench.counter_traffic() is None


def test_target_row_arithmetic():
    nbytes = 478_150_656
    target = nbytes / (0.7 * 8000.0 * 1e3)
    cold = np.array([target * 0.9, target * 0.95, target * 1.5])
    b2b = np.array([target * 1.1] * 4)
    rot = np.array([target * 0.99] * 5)
    row = bench._target_row("w", "op", 262144, 262144, nbytes, cold, b2b, rot, copies=3)
    assert row["target_us"] == pytest.approx(target)
    assert row["cold"]["median_us"] == pytest.approx(target * 0.95)
    assert row["cold"]["frac"] == pytest.approx(0.7 / 0.95)
    assert row["cold"]["GBps"] == pytest.approx(nbytes / (target * 0.95) / 1e3)
    assert row["meets_target"] == {"cold": True, "back_to_back": False, "cold_rotating": True}
    assert row["cold_rotating"]["copies"] == 3
    assert row["back_to_back"]["reps"] == 4


def test_threaded_oracle_run_equals_single_thread():
    from quantized_paged_kv_rope_amd import workloads as W

    case = W.prefill_262144(n=4096)
    n, sub_blocks = 3000, (3000 + 63) // 64
    _, backing1, out1 = bench._oracle_round_trip(case, n, sub_blocks, 1)
    _, backing4, out4 = bench._oracle_round_trip(case, n, sub_blocks, 4, chunk=256)
    assert np.array_equal(backing1, backing4)
    assert np.array_equal(out1, out4)
    # The sample covers whole pages from slot 0 and touched every record.
    assert backing1[: 64 * 512].any()
    assert out1.any()
