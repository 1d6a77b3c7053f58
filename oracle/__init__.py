"""fp64 CPU oracle for the varlen gated delta-rule hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product path (``gated_delta_rule_varlen_amd``) never imports it, and
this package imports nothing from the product path.  The arithmetic lives in ``gdn_oracle.c``
(plain C, fp64); this file only compiles it with gcc and marshals numpy arrays.

Dtype codes: 0 = float32, 1 = bfloat16 (raw uint16 bits), 2 = float16 (raw uint16 bits).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16, F16 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "bf16": BF16, "f16": F16}


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c into liboracle.so (gcc, -O2, OpenMP) and return its path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB_PATH)
            vp, i32, f64p = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_double)
            L.gdn_oracle_offsets_valid.argtypes = [vp, i32, i32]
            L.gdn_oracle_offsets_valid.restype = i32
            L.gdn_oracle_decode.argtypes = [vp, i32, ctypes.c_longlong]
            L.gdn_oracle_decode.restype = ctypes.c_double
            L.gdn_oracle_conv.argtypes = [i32] * 8 + [vp] * 7
            L.gdn_oracle_conv.restype = i32
            L.gdn_oracle_conv_capture.argtypes = [i32] * 5 + [vp] * 4
            L.gdn_oracle_conv_capture.restype = i32
            L.gdn_oracle_prepare.argtypes = [i32] * 10 + [vp] * 7
            L.gdn_oracle_prepare.restype = None
            L.gdn_oracle_scan.argtypes = [i32] * 13 + [ctypes.c_double] + [vp] * 11 + [i32, vp]
            L.gdn_oracle_scan.restype = i32
            L.gdn_oracle_threads.argtypes = []
            L.gdn_oracle_threads.restype = i32
            L.gdn_oracle_set_threads.argtypes = [i32]
            L.gdn_oracle_set_threads.restype = None
            del f64p
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _raw(a, code):
    """Check that a raw array matches its dtype code and make it C-contiguous."""
    if a is None:
        return None
    want = np.float32 if code == F32 else np.uint16
    if a.dtype != want:
        raise TypeError(f"expected {np.dtype(want)} storage for dtype code {code}, got {a.dtype}")
    return np.ascontiguousarray(a)


def offsets_valid(offsets, B, N) -> bool:
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    return bool(lib().gdn_oracle_offsets_valid(_ptr(off), int(B), int(N)))


def decode(raw, code) -> np.ndarray:
    """Decode raw storage (float32, or uint16 bits of bf16/f16) to float64 element by element."""
    raw = _raw(np.asarray(raw), code)
    flat = raw.reshape(-1)
    L = lib()
    return np.array([L.gdn_oracle_decode(_ptr(flat), code, i) for i in range(flat.size)],
                    dtype=np.float64).reshape(raw.shape)


def conv(x, w, offsets, *, W, D, x_dtype, bias=None, state_in=None, state_dtype=None, silu=False):
    """Varlen causal depthwise conv1d.  Returns (y [N,C] f64, state_out [B,C,L] f64) or None when
    the offsets are malformed (nothing written)."""
    xd = DTYPE_CODES[x_dtype]
    sd = DTYPE_CODES[state_dtype or x_dtype]
    x = _raw(x, xd)
    w = _raw(w, xd)
    bias = _raw(bias, xd)
    state_in = _raw(state_in, sd)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    N, C = x.shape
    B = off.size - 1
    L = (W - 1) * D
    y = np.zeros((N, C), np.float64)
    st = np.zeros((B, C, L), np.float64)
    rc = lib().gdn_oracle_conv(B, N, C, W, D, xd, sd, int(bool(silu)), _ptr(x), _ptr(w), _ptr(bias),
                               _ptr(state_in), _ptr(off), _ptr(y), _ptr(st))
    if rc == 1:
        return None
    assert rc == 0
    return y, st


def prepare(qkv, *, HQ, H, K, V, qkv_dtype, gate_dtype=None, a=None, b=None, A_log=None, dt_bias=None,
            l2norm=True, softplus=True, sigmoid=True):
    """q/k normalisation and gates.  Returns (qk [2,N,HQ,K] f64, gb [2,N,H] f64)."""
    qd = DTYPE_CODES[qkv_dtype]
    gd = DTYPE_CODES[gate_dtype or qkv_dtype]
    qkv = _raw(qkv, qd)
    a = _raw(a, gd)
    b = _raw(b, gd)
    A_log = None if A_log is None else np.ascontiguousarray(A_log, np.float32)
    dt_bias = None if dt_bias is None else np.ascontiguousarray(dt_bias, np.float32)
    N = qkv.shape[0]
    assert qkv.shape[1] == 2 * HQ * K + H * V
    qk = np.zeros((2, N, HQ, K), np.float64)
    gb = np.zeros((2, N, H), np.float64)
    lib().gdn_oracle_prepare(N, HQ, H, K, V, qd, gd, int(bool(l2norm)), int(bool(softplus)),
                             int(bool(sigmoid)), _ptr(qkv), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                             _ptr(qk), _ptr(gb))
    return qk, gb


def conv_capture(x, offsets, counts, *, cap, x_dtype):
    """Recorded conv inputs for speculative decoding: updates [B, cap, C] f64 (see the C source),
    or None when the offsets are malformed."""
    xd = DTYPE_CODES[x_dtype]
    x = _raw(x, xd)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    cnt = np.ascontiguousarray(counts, dtype=np.int32)
    N, C = x.shape
    B = off.size - 1
    upd = np.zeros((B, cap, C), np.float64)
    rc = lib().gdn_oracle_conv_capture(B, N, C, cap, xd, _ptr(x), _ptr(off), _ptr(cnt), _ptr(upd))
    return None if rc == 1 else upd


def scan(qkv, offsets, *, HQ, H, K, V, qkv_dtype, gate_dtype=None, a=None, b=None, A_log=None,
         dt_bias=None, state_in=None, l2norm=True, softplus=True, sigmoid=True, scale=0.0, retrieve=True,
         gate_per_key=False, counts=None, active=None, cap=0):
    """Gated delta-rule recurrence.  retrieve=False drops the retrieval term (the linear and gated
    update rules); gate_per_key=True takes a [N,H,K] decay input, one decay per key channel.  Returns (out [N,H,V] f64, state_out [B,H,V,K] f64), plus the capture capsule
    [B, cap*(H + HQ*K + H*V)] f64 when counts is given; None when the offsets are malformed."""
    qd = DTYPE_CODES[qkv_dtype]
    gd = DTYPE_CODES[gate_dtype or qkv_dtype]
    qkv = _raw(qkv, qd)
    a = _raw(a, gd)
    b = _raw(b, gd)
    A_log = None if A_log is None else np.ascontiguousarray(A_log, np.float32)
    dt_bias = None if dt_bias is None else np.ascontiguousarray(dt_bias, np.float32)
    state_in = None if state_in is None else np.ascontiguousarray(state_in, np.float32)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    N = qkv.shape[0]
    B = off.size - 1
    assert qkv.shape[1] == 2 * HQ * K + H * V
    out = np.zeros((N, H, V), np.float64)
    st = np.zeros((B, H, V, K), np.float64)
    capsule = cnt = act = None
    if counts is not None:
        cnt = np.ascontiguousarray(counts, dtype=np.int32)
        act = None if active is None else np.ascontiguousarray(active, dtype=np.int32)
        capsule = np.zeros((B, cap * (H + HQ * K + H * V)), np.float64)
    rc = lib().gdn_oracle_scan(B, N, HQ, H, K, V, qd, gd, int(bool(l2norm)), int(bool(softplus)),
                               int(bool(sigmoid)), int(bool(retrieve)), int(bool(gate_per_key)), float(scale),
                               _ptr(qkv), _ptr(a), _ptr(b),
                               _ptr(A_log), _ptr(dt_bias), _ptr(state_in), _ptr(off), _ptr(out), _ptr(st),
                               _ptr(cnt), _ptr(act), int(cap), _ptr(capsule))
    if rc == 1:
        return None
    if rc == 3:
        raise ValueError("a per-key-channel gate is not combined with a capture")
    if rc != 0:
        raise MemoryError("oracle scan could not allocate its buffers")
    return (out, st) if counts is None else (out, st, capsule)


def threads() -> int:
    return int(lib().gdn_oracle_threads())


def set_threads(n: int) -> None:
    """OpenMP threads of the following calls (for timing the oracle at a chosen width)."""
    lib().gdn_oracle_set_threads(int(n))
