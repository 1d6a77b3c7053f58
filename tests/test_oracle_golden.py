"""The oracle against a hand-derived worked example stored under tests/golden/ (CPU only)."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_k2v1.txt")


def _load():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    steps = np.array([[float(v) for v in r] for r in rows[:-1]])
    final = np.array([float(v) for v in rows[-1]])
    return steps, final


def test_worked_example_k2_v1():
    steps, final = _load()
    T = steps.shape[0]
    qkv = np.ascontiguousarray(steps[:, 0:5], dtype=np.float32)  # [q0 q1 | k0 k1 | v]
    a = np.ascontiguousarray(steps[:, 5:6], dtype=np.float32)
    b = np.ascontiguousarray(steps[:, 6:7], dtype=np.float32)
    out, st = oracle.scan(qkv, np.array([0, T], np.int32), HQ=1, H=1, K=2, V=1, qkv_dtype="f32", a=a, b=b,
                          l2norm=False, softplus=False, sigmoid=False, scale=1.0)
    assert np.array_equal(out[:, 0, 0], steps[:, 7])
    assert np.array_equal(st[0, 0, 0], final)
