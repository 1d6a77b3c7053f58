"""Host-side checks of bench.py that need no GPU: the one-GPU contract and the byte counts its
rooflines divide by."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_recurrence_bytes():
    # fp32 state read and written, bf16 token rows [q|k|v] and gates read, bf16 outputs written
    w = workloads.decode_step()
    state = 2 * 256 * 32 * 128 * 128 * 4
    tokens = 256 * ((2 * 16 * 128 + 32 * 128) * 2 + 2 * 32 * 2) + 256 * 32 * 128 * 2
    assert bench.scan_bytes(w) == state + tokens == 1080066048


def test_prepare_bytes():
    # q and k rows and two gate inputs read in bf16, fp32 q^/k^ and g/beta planes written
    w = workloads.varlen_prefill()
    per_token = 2 * 16 * 128 * 2 + 2 * 32 * 2 + (2 * 16 * 128 + 2 * 32) * 4
    assert bench.prepare_bytes(w) == w.N * per_token
