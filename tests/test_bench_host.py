"""Host-side logic of bench.py (no GPU): algorithmic byte counts and the
one-GPU guard."""
import os
import subprocess
import sys

import bench
from scan_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_alg_bytes_lm_diag():
    # per token-head: q, k, v bf16 (3*128*2) + a fp32 (128*4) + r (4) + o bf16 (128*2) = 1540 B;
    # per sequence: lT (128*4) + etaT (128*128*4) = 66048 B
    w = gen.WORKLOADS["lm_diag"]
    assert bench.alg_bytes(w) == 1540 * 8 * 16 * 2048 + 66048 * 8 * 16


def test_alg_bytes_prefill_counts_the_state_both_ways():
    # iso, per token-head: q, k, v bf16 (3*64*2) + a, qn, r (12) + o bf16 (64*2) = 524 B;
    # per sequence: l and eta read (4 + 64*64*4) and written (the same)
    w = gen.PREFILL
    assert bench.prefill_alg_bytes(w) == 524 * 256 * 32 * 16 + 2 * (4 + 64 * 64 * 4) * 256 * 32


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
