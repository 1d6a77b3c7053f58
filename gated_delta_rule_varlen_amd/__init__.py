"""MI355X (gfx950) varlen gated delta-rule hot path.

A thin binding over libgdn's C ABI (include/gdn.h).  These functions only marshal arguments: they
check that tensors are device-resident and contiguous, allocate outputs with torch when the
caller does not pass them, and hand raw device pointers plus torch's current HIP stream to the
library.  Every step of the computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _abi
from ._abi import GdnError, PATH_NAMES, lib  # noqa: F401

__all__ = ["conv1d_varlen", "conv1d_varlen_capture", "prepare_qk_gates", "prepare_qk_gates_strided", "scan_varlen",
           "scan_varlen_capture", "scan_varlen_strided", "scan_varlen_noalloc", "scan_workspace_bytes", "decode_step", "GdnError", "lib"]

_DTYPE = {torch.float32: _abi.F32, torch.bfloat16: _abi.BF16, torch.float16: _abi.F16}
_TORCH = {v: k for k, v in _DTYPE.items()}


def _code(t: torch.Tensor, what: str) -> int:
    if t.dtype not in _DTYPE:
        raise TypeError(f"{what}: unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


def _ptr(t: Optional[torch.Tensor], what: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _row_view(t: Optional[torch.Tensor], width: int, what: str):
    """(device pointer, row stride in elements) of a [N, ...] tensor whose rows are contiguous
    blocks of `width` elements; the row stride itself is free."""
    if t is None:
        return None, width
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if t.shape[0] == 0:
        return ctypes.c_void_p(t.data_ptr()), width
    # [N, heads, width] with each token's block contiguous merges into a [N, heads*width] view
    rows = t.reshape(t.shape[0], -1) if t.dim() > 2 and t[0].is_contiguous() else t
    if rows.dim() != 2 or rows.shape[1] != width or (rows.shape[0] > 1 and rows.stride(1) != 1):
        raise ValueError(f"{what} must be [N, {width}] (or [N, heads, width]) with contiguous rows")
    return ctypes.c_void_p(rows.data_ptr()), rows.stride(0) if rows.shape[0] > 1 else width


def _streams(q, k, v, HQ, H, K, V):
    qp, qs = _row_view(q, HQ * K, "q")
    kp, ks = _row_view(k, HQ * K, "k")
    vp, vs = _row_view(v, H * V, "v")
    return _abi.QKVStreams(qp, kp, vp, qs, ks, vs)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, where: str):
    if status != _abi.OK:
        raise GdnError(status, where)


def conv1d_varlen(x: torch.Tensor, weight: torch.Tensor, offsets: torch.Tensor, *, bias=None, state_in=None,
                  dilation: int = 1, silu: bool = False, state_dtype=None, y=None, state_out=None,
                  write_state: bool = True, dev_status=None):
    """Varlen depthwise causal conv1d with a carried window (gdn_conv1d_varlen).

    x [N, C]; weight [C, W] (or [C, 1, W]); offsets int32 [B+1]; bias [C] or None; state_in
    [B, C, (W-1)*dilation] or None (zeros).  Returns (y [N, C], state_out or None).  Pass
    state_out=state_in for an in-place window update."""
    if weight.dim() == 3:
        weight = weight.reshape(weight.shape[0], weight.shape[2])
    N, C = x.shape
    W = weight.shape[1]
    B = offsets.numel() - 1
    L = (W - 1) * dilation
    if state_dtype is None:
        state_dtype = state_in.dtype if state_in is not None else (state_out.dtype if state_out is not None else x.dtype)
    if y is None:
        y = torch.empty_like(x)
    if state_out is None and write_state and L > 0:
        state_out = torch.empty((B, C, L), dtype=state_dtype, device=x.device)
    d = _abi.ConvDesc(B, N, C, W, dilation, _code(x, "x"), _DTYPE[state_dtype], _abi.CONV_SILU if silu else 0)
    st = lib().gdn_conv1d_varlen(ctypes.byref(d), _ptr(x, "x"), _ptr(weight, "weight"), _ptr(bias, "bias"),
                                 _ptr(state_in, "state_in"), _ptr(y, "y"), _ptr(state_out, "state_out"),
                                 _ptr(offsets, "offsets"), _ptr(dev_status, "dev_status"), _stream(x.device))
    _check(st, "gdn_conv1d_varlen")
    return y, state_out


def conv1d_varlen_capture(x: torch.Tensor, weight: torch.Tensor, offsets: torch.Tensor, *, cap: int,
                          counts: torch.Tensor, updates=None, bias=None, state_in=None, dilation: int = 1,
                          silu: bool = False, state_dtype=None, y=None, state_out=None, write_state: bool = True,
                          dev_status=None):
    """conv1d_varlen that also records the first min(counts[b], cap, len) input rows of each sequence
    (gdn_conv1d_varlen_capture).  counts int32 [B].  Returns (y, state_out, updates [B, cap, C])."""
    if weight.dim() == 3:
        weight = weight.reshape(weight.shape[0], weight.shape[2])
    N, C = x.shape
    W = weight.shape[1]
    B = offsets.numel() - 1
    L = (W - 1) * dilation
    if state_dtype is None:
        state_dtype = state_in.dtype if state_in is not None else (state_out.dtype if state_out is not None else x.dtype)
    if y is None:
        y = torch.empty_like(x)
    if state_out is None and write_state and L > 0:
        state_out = torch.empty((B, C, L), dtype=state_dtype, device=x.device)
    if updates is None:
        updates = torch.empty((B, cap, C), dtype=x.dtype, device=x.device)
    d = _abi.ConvDesc(B, N, C, W, dilation, _code(x, "x"), _DTYPE[state_dtype], _abi.CONV_SILU if silu else 0)
    st = lib().gdn_conv1d_varlen_capture(ctypes.byref(d), _ptr(x, "x"), _ptr(weight, "weight"), _ptr(bias, "bias"),
                                         _ptr(state_in, "state_in"), _ptr(y, "y"), _ptr(state_out, "state_out"),
                                         _ptr(offsets, "offsets"), int(cap), _ptr(counts, "counts"),
                                         _ptr(updates, "updates"), _ptr(dev_status, "dev_status"), _stream(x.device))
    _check(st, "gdn_conv1d_varlen_capture")
    return y, state_out, updates


def _scan_desc(qkv, B, HQ, H, K, V, gate, l2norm, softplus, sigmoid, scale, path, retrieve=True,
               gate_per_key=False):
    flags = (_abi.L2NORM if l2norm else 0) | (_abi.SOFTPLUS if softplus else 0) | (_abi.SIGMOID if sigmoid else 0)
    flags |= (0 if retrieve else _abi.NO_RETRIEVE) | (_abi.GATE_PER_KEY if gate_per_key else 0)
    qd = _code(qkv, "qkv")
    gd = _code(gate, "gate inputs") if gate is not None else qd
    return _abi.ScanDesc(B, qkv.shape[0], HQ, H, K, V, qd, gd, flags, float(scale), _abi.PATH_CODES[path])


def prepare_qk_gates(qkv: torch.Tensor, *, HQ: int, H: int, K: int, V: int, a=None, b=None, A_log=None,
                     dt_bias=None, l2norm=True, softplus=True, sigmoid=True, qk_out=None, gb_out=None):
    """q/k normalisation and gate/rate activations (gdn_prepare_qk_gates).
    Returns (qk [2, N, HQ, K] fp32, gb [2, N, H] fp32)."""
    N = qkv.shape[0]
    if qk_out is None:
        qk_out = torch.empty((2, N, HQ, K), dtype=torch.float32, device=qkv.device)
    if gb_out is None:
        gb_out = torch.empty((2, N, H), dtype=torch.float32, device=qkv.device)
    d = _scan_desc(qkv, 1, HQ, H, K, V, a if a is not None else b, l2norm, softplus, sigmoid, 0.0, "auto")
    st = lib().gdn_prepare_qk_gates(ctypes.byref(d), _ptr(qkv, "qkv"), _ptr(a, "a"), _ptr(b, "b"),
                                    _ptr(A_log, "A_log"), _ptr(dt_bias, "dt_bias"), _ptr(qk_out, "qk_out"),
                                    _ptr(gb_out, "gb_out"), _stream(qkv.device))
    _check(st, "gdn_prepare_qk_gates")
    return qk_out, gb_out


def prepare_qk_gates_strided(q: torch.Tensor, k: torch.Tensor, *, HQ: int, H: int, K: int, V: int, a=None, b=None,
                             A_log=None, dt_bias=None, l2norm=True, softplus=True, sigmoid=True, qk_out=None,
                             gb_out=None):
    """prepare_qk_gates on separate q and k token streams (gdn_prepare_qk_gates_strided): q, k are
    [N, HQ, K] or [N, HQ*K] with contiguous rows and any row stride."""
    N = q.shape[0]
    if qk_out is None:
        qk_out = torch.empty((2, N, HQ, K), dtype=torch.float32, device=q.device)
    if gb_out is None:
        gb_out = torch.empty((2, N, H), dtype=torch.float32, device=q.device)
    d = _scan_desc(q, 1, HQ, H, K, V, a if a is not None else b, l2norm, softplus, sigmoid, 0.0, "auto")
    s = _streams(q, k, None, HQ, H, K, V)
    st = lib().gdn_prepare_qk_gates_strided(ctypes.byref(d), ctypes.byref(s), _ptr(a, "a"), _ptr(b, "b"),
                                            _ptr(A_log, "A_log"), _ptr(dt_bias, "dt_bias"), _ptr(qk_out, "qk_out"),
                                            _ptr(gb_out, "gb_out"), _stream(q.device))
    _check(st, "gdn_prepare_qk_gates_strided")
    return qk_out, gb_out


def scan_workspace_bytes(qkv: torch.Tensor, B: int, *, HQ, H, K, V, l2norm=True, softplus=True, sigmoid=True,
                         path="auto", gate_dtype=None) -> int:
    d = _scan_desc(qkv, B, HQ, H, K, V, None, l2norm, softplus, sigmoid, 0.0, path)
    if gate_dtype is not None:
        d.gate_dtype = _DTYPE[gate_dtype]
    n = ctypes.c_size_t(0)
    _check(lib().gdn_scan_workspace_bytes(ctypes.byref(d), ctypes.byref(n)), "gdn_scan_workspace_bytes")
    return int(n.value)


def scan_varlen(qkv: torch.Tensor, offsets: torch.Tensor, *, HQ: int, H: int, K: int, V: int, a=None, b=None,
                A_log=None, dt_bias=None, state_in=None, qk_prep=None, gb_prep=None, l2norm=True, softplus=True,
                sigmoid=True, scale: float = 0.0, path: str = "auto", out=None, state_out=None,
                write_state: bool = True, workspace=None, dev_status=None, retrieve: bool = True,
                gate_per_key: bool = False):
    """Gated delta-rule recurrence over offset-packed sequences (gdn_scan_varlen).  retrieve=False
    selects the linear/gated update rules (no retrieval term); gate_per_key=True takes a [N, H, K]
    decay input, one decay per key channel.
    Returns (out [N, H, V], state_out [B, H, V, K] fp32 or None, path name that ran)."""
    N = qkv.shape[0]
    B = offsets.numel() - 1
    if out is None:
        out = torch.empty((N, H, V), dtype=qkv.dtype, device=qkv.device)
    if state_out is None and write_state:
        state_out = torch.empty((B, H, V, K), dtype=torch.float32, device=qkv.device)
    d = _scan_desc(qkv, B, HQ, H, K, V, a if a is not None else b, l2norm, softplus, sigmoid, scale, path, retrieve,
                   gate_per_key)
    if workspace is None and path in ("auto", "chunk"):
        n = ctypes.c_size_t(0)
        _check(lib().gdn_scan_workspace_bytes(ctypes.byref(d), ctypes.byref(n)), "gdn_scan_workspace_bytes")
        if n.value:
            workspace = torch.empty(int(n.value), dtype=torch.uint8, device=qkv.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    used = ctypes.c_int32(-1)
    st = lib().gdn_scan_varlen(ctypes.byref(d), _ptr(qkv, "qkv"), _ptr(qk_prep, "qk_prep"), _ptr(gb_prep, "gb_prep"),
                               _ptr(a, "a"), _ptr(b, "b"), _ptr(A_log, "A_log"), _ptr(dt_bias, "dt_bias"),
                               _ptr(state_in, "state_in"), _ptr(out, "out"), _ptr(state_out, "state_out"),
                               _ptr(offsets, "offsets"), _ptr(workspace, "workspace"), ws_bytes,
                               _ptr(dev_status, "dev_status"), ctypes.byref(used), _stream(qkv.device))
    _check(st, "gdn_scan_varlen")
    return out, state_out, PATH_NAMES.get(used.value, str(used.value))


def scan_varlen_noalloc(qkv: torch.Tensor, offsets: torch.Tensor, *, HQ: int, H: int, K: int, V: int, a=None, b=None,
                        A_log=None, dt_bias=None, state_in=None, qk_prep=None, gb_prep=None, l2norm=True,
                        softplus=True, sigmoid=True, scale: float = 0.0, path: str = "auto", out=None,
                        state_out=None, dev_status=None, retrieve: bool = True, gate_per_key: bool = False):
    """scan_varlen without a workspace argument (gdn_scan_varlen_noalloc): the chunked path's
    workspace is the library's own device array, so the call allocates no device memory when out
    and state_out are given.  Returns (out, state_out, path name that ran)."""
    N = qkv.shape[0]
    B = offsets.numel() - 1
    if out is None:
        out = torch.empty((N, H, V), dtype=qkv.dtype, device=qkv.device)
    if state_out is None:
        state_out = torch.empty((B, H, V, K), dtype=torch.float32, device=qkv.device)
    d = _scan_desc(qkv, B, HQ, H, K, V, a if a is not None else b, l2norm, softplus, sigmoid, scale, path, retrieve,
                   gate_per_key)
    used = ctypes.c_int32(-1)
    st = lib().gdn_scan_varlen_noalloc(ctypes.byref(d), _ptr(qkv, "qkv"), _ptr(qk_prep, "qk_prep"),
                                       _ptr(gb_prep, "gb_prep"), _ptr(a, "a"), _ptr(b, "b"), _ptr(A_log, "A_log"),
                                       _ptr(dt_bias, "dt_bias"), _ptr(state_in, "state_in"), _ptr(out, "out"),
                                       _ptr(state_out, "state_out"), _ptr(offsets, "offsets"),
                                       _ptr(dev_status, "dev_status"), ctypes.byref(used), _stream(qkv.device))
    _check(st, "gdn_scan_varlen_noalloc")
    return out, state_out, PATH_NAMES.get(used.value, str(used.value))


def scan_varlen_strided(q, k, v, offsets: torch.Tensor, *, HQ: int, H: int, K: int, V: int, a=None, b=None,
                        A_log=None, dt_bias=None, state_in=None, qk_prep=None, gb_prep=None, l2norm=True,
                        softplus=True, sigmoid=True, scale: float = 0.0, path: str = "auto", out=None, state_out=None,
                        write_state: bool = True, workspace=None, dev_status=None, retrieve: bool = True,
                        gate_per_key: bool = False):
    """scan_varlen on separate token streams (gdn_scan_varlen_strided): q, k [N, HQ, K] (or
    [N, HQ*K]) and v [N, H, V] (or [N, H*V]), each with contiguous rows and any row stride; q and k
    may be None with prepared inputs.  Returns (out, state_out, path name that ran)."""
    N = v.shape[0]
    B = offsets.numel() - 1
    if out is None:
        out = torch.empty((N, H, V), dtype=v.dtype, device=v.device)
    if state_out is None and write_state:
        state_out = torch.empty((B, H, V, K), dtype=torch.float32, device=v.device)
    d = _scan_desc(v, B, HQ, H, K, V, a if a is not None else b, l2norm, softplus, sigmoid, scale, path, retrieve,
                   gate_per_key)
    d.N = N
    if workspace is None and path in ("auto", "chunk"):
        n = ctypes.c_size_t(0)
        _check(lib().gdn_scan_workspace_bytes(ctypes.byref(d), ctypes.byref(n)), "gdn_scan_workspace_bytes")
        if n.value:
            workspace = torch.empty(int(n.value), dtype=torch.uint8, device=v.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    s = _streams(q, k, v, HQ, H, K, V)
    used = ctypes.c_int32(-1)
    st = lib().gdn_scan_varlen_strided(ctypes.byref(d), ctypes.byref(s), _ptr(qk_prep, "qk_prep"),
                                       _ptr(gb_prep, "gb_prep"), _ptr(a, "a"), _ptr(b, "b"), _ptr(A_log, "A_log"),
                                       _ptr(dt_bias, "dt_bias"), _ptr(state_in, "state_in"), _ptr(out, "out"),
                                       _ptr(state_out, "state_out"), _ptr(offsets, "offsets"),
                                       _ptr(workspace, "workspace"), ws_bytes, _ptr(dev_status, "dev_status"),
                                       ctypes.byref(used), _stream(v.device))
    _check(st, "gdn_scan_varlen_strided")
    return out, state_out, PATH_NAMES.get(used.value, str(used.value))


def capsule_width(cap: int, *, HQ: int, H: int, K: int, V: int) -> int:
    """Row width of the fp32 capture capsule: cap * (H + HQ*K + H*V)."""
    return cap * (H + HQ * K + H * V)


def scan_varlen_capture(qkv: torch.Tensor, offsets: torch.Tensor, *, cap: int, counts: torch.Tensor, HQ: int, H: int,
                        K: int, V: int, active=None, capsule=None, a=None, b=None, A_log=None, dt_bias=None,
                        state_in=None, qk_prep=None, gb_prep=None, l2norm=True, softplus=True, sigmoid=True,
                        scale: float = 0.0, path: str = "auto", out=None, state_out=None, write_state: bool = True,
                        workspace=None, dev_status=None, retrieve: bool = True):
    """scan_varlen that also records g, k^ and delta of the first min(counts[b], cap, len) tokens of
    each sequence (gdn_scan_varlen_capture); active int32 [1] or None.  The workspace is allocated as
    in scan_varlen when absent.
    Returns (out, state_out, capsule [B, cap*(H + HQ*K + H*V)] fp32, path name that ran)."""
    N = qkv.shape[0]
    B = offsets.numel() - 1
    if out is None:
        out = torch.empty((N, H, V), dtype=qkv.dtype, device=qkv.device)
    if state_out is None and write_state:
        state_out = torch.empty((B, H, V, K), dtype=torch.float32, device=qkv.device)
    if capsule is None:
        capsule = torch.empty((B, capsule_width(cap, HQ=HQ, H=H, K=K, V=V)), dtype=torch.float32, device=qkv.device)
    d = _scan_desc(qkv, B, HQ, H, K, V, a if a is not None else b, l2norm, softplus, sigmoid, scale, path, retrieve)
    if workspace is None and path in ("auto", "chunk"):
        n = ctypes.c_size_t(0)
        _check(lib().gdn_scan_workspace_bytes(ctypes.byref(d), ctypes.byref(n)), "gdn_scan_workspace_bytes")
        if n.value > 0:
            workspace = torch.empty(int(n.value), dtype=torch.uint8, device=qkv.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    used = ctypes.c_int32(-1)
    st = lib().gdn_scan_varlen_capture(ctypes.byref(d), _ptr(qkv, "qkv"), _ptr(qk_prep, "qk_prep"),
                                       _ptr(gb_prep, "gb_prep"), _ptr(a, "a"), _ptr(b, "b"), _ptr(A_log, "A_log"),
                                       _ptr(dt_bias, "dt_bias"), _ptr(state_in, "state_in"), _ptr(out, "out"),
                                       _ptr(state_out, "state_out"), _ptr(offsets, "offsets"), int(cap),
                                       _ptr(counts, "counts"), _ptr(active, "active"), _ptr(capsule, "capsule"),
                                       _ptr(workspace, "workspace"), ws_bytes, _ptr(dev_status, "dev_status"),
                                       ctypes.byref(used), _stream(qkv.device))
    _check(st, "gdn_scan_varlen_capture")
    return out, state_out, capsule, PATH_NAMES.get(used.value, str(used.value))


def decode_step(x: torch.Tensor, weight: torch.Tensor, offsets: torch.Tensor, *, HQ: int, H: int, K: int, V: int,
                bias=None, conv_state_in=None, conv_state_out=None, dilation: int = 1, silu: bool = True,
                conv_state_dtype=None, a=None, b=None, A_log=None, dt_bias=None, state_in=None, state_out=None,
                l2norm=True, softplus=True, sigmoid=True, scale: float = 0.0, out=None, write_state: bool = True,
                dev_status=None, retrieve: bool = True):
    """A decode step in one launch (gdn_decode_step): conv1d_varlen over x followed by scan_varlen over
    its output on the DECODE path, for at most one token per sequence.  Pass conv_state_out=conv_state_in
    and state_out=state_in for in-place updates.  Returns (out [N, H, V], state_out, conv_state_out)."""
    if weight.dim() == 3:
        weight = weight.reshape(weight.shape[0], weight.shape[2])
    N, C = x.shape
    W = weight.shape[1]
    B = offsets.numel() - 1
    L = (W - 1) * dilation
    if conv_state_dtype is None:
        src = conv_state_in if conv_state_in is not None else conv_state_out
        conv_state_dtype = src.dtype if src is not None else x.dtype
    if out is None:
        out = torch.empty((N, H, V), dtype=x.dtype, device=x.device)
    if state_out is None and write_state:
        state_out = torch.empty((B, H, V, K), dtype=torch.float32, device=x.device)
    if conv_state_out is None and write_state and L > 0:
        conv_state_out = torch.empty((B, C, L), dtype=conv_state_dtype, device=x.device)
    cd = _abi.ConvDesc(B, N, C, W, dilation, _code(x, "x"), _DTYPE[conv_state_dtype], _abi.CONV_SILU if silu else 0)
    sd = _scan_desc(x, B, HQ, H, K, V, a if a is not None else b, l2norm, softplus, sigmoid, scale, "decode",
                    retrieve)
    st = lib().gdn_decode_step(ctypes.byref(cd), ctypes.byref(sd), _ptr(x, "x"), _ptr(weight, "weight"),
                               _ptr(bias, "bias"), _ptr(conv_state_in, "conv_state_in"),
                               _ptr(conv_state_out, "conv_state_out"), _ptr(a, "a"), _ptr(b, "b"),
                               _ptr(A_log, "A_log"), _ptr(dt_bias, "dt_bias"), _ptr(state_in, "state_in"),
                               _ptr(out, "out"), _ptr(state_out, "state_out"), _ptr(offsets, "offsets"),
                               _ptr(dev_status, "dev_status"), _stream(x.device))
    _check(st, "gdn_decode_step")
    return out, state_out, conv_state_out
