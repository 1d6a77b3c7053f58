"""The C-ABI library on the host (CPU only): it loads, exports every symbol include/gdn.h declares,
and rejects bad arguments with the documented status codes before launching anything.

Only argument sets that fail host validation are passed here, so no call reaches the HIP runtime;
device pointers are stand-in addresses that are never dereferenced."""
import ctypes
import os
import re

import pytest

from gpu_util import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def abi():
    ensure_built()
    from gated_delta_rule_varlen_amd import _abi

    _abi.lib()
    return _abi


def test_header_declarations_are_all_exported(abi):
    header = open(os.path.join(ROOT, "include", "gdn.h")).read()
    declared = set(re.findall(r"^\s*(?:gdn_status|const char \*|int)\s*(gdn_\w+)\s*\(", header, re.M))
    assert declared == set(abi.EXPORTS)
    for name in declared:
        assert hasattr(abi.lib(), name), name


def test_version_and_status_strings(abi):
    assert abi.lib().gdn_abi_version() == 4
    for code in range(0, -10, -1):
        assert abi.status_string(code) and abi.status_string(code) != "unknown status"
    assert abi.status_string(-99) == "unknown status"


P = 0x10000  # a 16-byte-aligned stand-in device address (never dereferenced here)


def conv(abi, desc, x=P, w=P, bias=None, sin=None, y=P, sout=None, off=P):
    return abi.lib().gdn_conv1d_varlen(ctypes.byref(desc), x, w, bias, sin, y, sout, off, None, None)


@pytest.mark.parametrize(
    "fields,kw,want",
    [
        (dict(B=0), {}, "ERR_SHAPE"),
        (dict(N=-1), {}, "ERR_SHAPE"),
        (dict(C=0), {}, "ERR_SHAPE"),
        (dict(W=0), {}, "ERR_SHAPE"),
        (dict(D=0), {}, "ERR_SHAPE"),
        (dict(x_dtype=7), {}, "ERR_DTYPE"),
        (dict(x_dtype=0, state_dtype=1), {}, "ERR_DTYPE"),
        (dict(flags=2), {}, "ERR_UNSUPPORTED"),
        (dict(D=2**30), {}, "ERR_OVERFLOW"),
        ({}, dict(w=None), "ERR_NULL"),
        ({}, dict(off=None), "ERR_NULL"),
        ({}, dict(x=None), "ERR_NULL"),
        ({}, dict(y=None), "ERR_NULL"),
        ({}, dict(x=P + 8), "ERR_ALIGN"),
        ({}, dict(sin=P + 4), "ERR_ALIGN"),
    ],
)
def test_conv_host_validation(abi, fields, kw, want):
    base = dict(B=2, N=64, C=192, W=4, D=1, x_dtype=0, state_dtype=0, flags=0)
    base.update(fields)
    assert conv(abi, abi.ConvDesc(**base), **kw) == getattr(abi, want)


def scan_desc(abi, **fields):
    base = dict(B=2, N=64, HQ=2, H=2, K=32, V=32, qkv_dtype=0, gate_dtype=0, flags=7, scale=0.0, path=0)
    base.update(fields)
    return abi.ScanDesc(**base)


def scan(abi, d, qkv=P, qk=None, gb=None, a=None, b=None, alog=None, dtb=None, sin=None, out=P, sout=None, off=P,
         ws=None, ws_bytes=0):
    return abi.lib().gdn_scan_varlen(ctypes.byref(d), qkv, qk, gb, a, b, alog, dtb, sin, out, sout, off, ws,
                                     ws_bytes, None, None, None)


@pytest.mark.parametrize(
    "fields,kw,want",
    [
        (dict(B=0), {}, "ERR_SHAPE"),
        (dict(HQ=3, H=4), {}, "ERR_SHAPE"),  # H % HQ != 0
        (dict(K=512), {}, "ERR_SHAPE"),  # the pages' limit: K <= 256
        (dict(V=0), {}, "ERR_SHAPE"),
        (dict(qkv_dtype=5), {}, "ERR_DTYPE"),
        (dict(qkv_dtype=1, gate_dtype=2), {}, "ERR_DTYPE"),
        (dict(flags=32), {}, "ERR_UNSUPPORTED"),
        (dict(path=9), {}, "ERR_UNSUPPORTED"),
        # the chunked form needs the retrieval term: shape and dtype eligible, GDN_NO_RETRIEVE set
        (dict(qkv_dtype=1, gate_dtype=1, K=64, V=64, flags=7 | 8, path=3), dict(a=P, alog=P, dtb=P), "ERR_UNSUPPORTED"),
        (dict(path=3), {}, "ERR_UNSUPPORTED"),  # chunked path not eligible here
        (dict(qkv_dtype=1, gate_dtype=1, V=33, H=2), {}, "ERR_ALIGN"),  # token row not a multiple of 16 bytes
        (dict(HQ=2**22, H=2**22, K=256, V=1), {}, "ERR_OVERFLOW"),
        ({}, dict(qkv=None), "ERR_NULL"),
        ({}, dict(out=None), "ERR_NULL"),
        ({}, dict(off=None), "ERR_NULL"),
        ({}, dict(qk=P), "ERR_NULL"),  # prepared inputs come in pairs
        ({}, dict(a=P), "ERR_NULL"),  # softplus needs A_log and dt_bias
        ({}, dict(out=P + 2), "ERR_ALIGN"),
        ({}, dict(sin=P + 8), "ERR_ALIGN"),
    ],
)
def test_scan_host_validation(abi, fields, kw, want):
    assert scan(abi, scan_desc(abi, **fields), **kw) == getattr(abi, want)


def decode_step(abi, cfields=None, sfields=None, x=P, w=P, out=P, off=P, a=None, alog=None, dtb=None, sin=None,
                sout=None, csin=None, csout=None):
    cbase = dict(B=4, N=4, C=192, W=4, D=1, x_dtype=0, state_dtype=0, flags=1)
    cbase.update(cfields or {})
    sbase = dict(B=4, N=4, HQ=2, H=2, K=32, V=32, qkv_dtype=0, gate_dtype=0, flags=7, scale=0.0, path=0)
    sbase.update(sfields or {})
    cd, sd = abi.ConvDesc(**cbase), abi.ScanDesc(**sbase)
    return abi.lib().gdn_decode_step(ctypes.byref(cd), ctypes.byref(sd), x, w, None, csin, csout, a, None, alog, dtb,
                                     sin, out, sout, off, None, None)


@pytest.mark.parametrize(
    "cf,sf,kw,want",
    [
        (dict(C=200), {}, {}, "ERR_SHAPE"),  # conv width != 2*HQ*K + H*V
        (dict(B=3), {}, {}, "ERR_SHAPE"),  # descriptors disagree
        (dict(N=3), {}, {}, "ERR_SHAPE"),
        (dict(x_dtype=1, state_dtype=1), {}, {}, "ERR_DTYPE"),  # conv and scan dtypes differ
        (dict(N=5), dict(N=5), {}, "ERR_UNSUPPORTED"),  # more tokens than sequences: not a decode step
        ({}, dict(path=2), {}, "ERR_UNSUPPORTED"),  # SEQ requested
        (dict(W=6), {}, {}, "ERR_UNSUPPORTED"),  # (W-1)*D > 4
        (dict(W=3, D=3), {}, {}, "ERR_UNSUPPORTED"),
        (dict(W=9), {}, {}, "ERR_UNSUPPORTED"),
        (dict(flags=4), {}, {}, "ERR_UNSUPPORTED"),
        (dict(C=4 * 32 + 2 * 30), dict(V=30), {}, "ERR_UNSUPPORTED"),  # V % 4 != 0
        (dict(C=2 * 2 * 48 + 2 * 32), dict(K=48), {}, "ERR_UNSUPPORTED"),  # a width the fused step does not take
        ({}, dict(HQ=3), {}, "ERR_SHAPE"),
        ({}, {}, dict(w=None), "ERR_NULL"),
        ({}, {}, dict(off=None), "ERR_NULL"),
        ({}, {}, dict(x=None), "ERR_NULL"),
        ({}, {}, dict(out=None), "ERR_NULL"),
        ({}, {}, dict(a=P), "ERR_NULL"),  # softplus needs A_log and dt_bias
        ({}, {}, dict(x=P + 2), "ERR_ALIGN"),
        ({}, {}, dict(csin=P + 4), "ERR_ALIGN"),
        ({}, {}, dict(sout=P + 8), "ERR_ALIGN"),
    ],
)
def test_decode_step_host_validation(abi, cf, sf, kw, want):
    assert decode_step(abi, cf, sf, **kw) == getattr(abi, want)


def test_decode_step_rejects_missing_descriptor(abi):
    sd = scan_desc(abi)
    assert abi.lib().gdn_decode_step(None, ctypes.byref(sd), *([P] * 2), *([None] * 13)) == abi.ERR_NULL


def test_prepare_host_validation(abi):
    L = abi.lib()
    d = scan_desc(abi)
    assert L.gdn_prepare_qk_gates(ctypes.byref(d), P, None, None, None, None, None, None, None) == abi.ERR_NULL
    assert L.gdn_prepare_qk_gates(ctypes.byref(d), P, P, None, None, None, P, P, None) == abi.ERR_NULL
    assert L.gdn_prepare_qk_gates(ctypes.byref(d), P, None, None, None, None, P + 4, P, None) == abi.ERR_ALIGN
    bad = scan_desc(abi, K=300)
    assert L.gdn_prepare_qk_gates(ctypes.byref(bad), P, None, None, None, None, P, P, None) == abi.ERR_SHAPE
    # a call without tokens writes nothing, so it needs no buffers at all (and launches nothing)
    empty = scan_desc(abi, N=0)
    assert L.gdn_prepare_qk_gates(ctypes.byref(empty), None, None, None, None, None, None, None, None) == abi.OK


def test_workspace_query(abi):
    n = ctypes.c_size_t(123)
    d = scan_desc(abi, path=2)
    assert abi.lib().gdn_scan_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == abi.OK and n.value == 0
    assert abi.lib().gdn_scan_workspace_bytes(ctypes.byref(d), None) == abi.ERR_NULL
    assert abi.lib().gdn_scan_workspace_bytes(None, ctypes.byref(n)) == abi.ERR_NULL


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from gated_delta_rule_varlen_amd import _abi

    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "libgdn.so"))
    with pytest.raises(ImportError):
        _abi.lib()


def conv_capture(abi, desc, cap=4, counts=P, updates=P, **kw):
    x, w, y, off = kw.get("x", P), kw.get("w", P), kw.get("y", P), kw.get("off", P)
    return abi.lib().gdn_conv1d_varlen_capture(ctypes.byref(desc), x, w, None, None, y, None, off, cap, counts,
                                               updates, None, None)


@pytest.mark.parametrize(
    "fields,kw,want",
    [
        ({}, dict(cap=0), "ERR_SHAPE"),
        ({}, dict(cap=-3), "ERR_SHAPE"),
        ({}, dict(counts=None), "ERR_NULL"),
        ({}, dict(updates=None), "ERR_NULL"),
        ({}, dict(updates=P + 2), "ERR_ALIGN"),
        ({}, dict(cap=2**24), "ERR_OVERFLOW"),  # cap * C beyond int32
        (dict(D=0), {}, "ERR_SHAPE"),  # the conv's own checks still apply
        ({}, dict(x=None), "ERR_NULL"),
    ],
)
def test_conv_capture_host_validation(abi, fields, kw, want):
    base = dict(B=2, N=64, C=192, W=4, D=1, x_dtype=0, state_dtype=0, flags=0)
    base.update(fields)
    assert conv_capture(abi, abi.ConvDesc(**base), **kw) == getattr(abi, want)


def scan_capture(abi, d, cap=4, counts=P, active=None, capsule=P, qkv=P, out=P, off=P):
    return abi.lib().gdn_scan_varlen_capture(ctypes.byref(d), qkv, None, None, None, None, None, None, None, out,
                                             None, off, cap, counts, active, capsule, None, 0, None, None, None)


@pytest.mark.parametrize(
    "fields,kw,want",
    [
        ({}, dict(cap=0), "ERR_SHAPE"),
        ({}, dict(counts=None), "ERR_NULL"),
        ({}, dict(capsule=None), "ERR_NULL"),
        ({}, dict(capsule=P + 4), "ERR_ALIGN"),
        ({}, dict(cap=2**24), "ERR_OVERFLOW"),  # the capsule row width must be an int32
        (dict(path=3), {}, "ERR_UNSUPPORTED"),  # a shape the chunked form does not take
        (dict(K=512), {}, "ERR_SHAPE"),  # the recurrence's own checks still apply
        ({}, dict(off=None), "ERR_NULL"),
        ({}, dict(out=None), "ERR_NULL"),
    ],
)
def test_scan_capture_host_validation(abi, fields, kw, want):
    assert scan_capture(abi, scan_desc(abi, **fields), **kw) == getattr(abi, want)


def test_per_key_gate_host_validation(abi):
    """GDN_GATE_PER_KEY runs on fused inputs through the token-sequential paths only."""
    L = abi.lib()
    pk = 7 | 16
    d = scan_desc(abi, flags=pk)
    assert L.gdn_prepare_qk_gates(ctypes.byref(d), P, P, None, P, P, P, P, None) == abi.ERR_UNSUPPORTED
    assert scan(abi, d, qk=P, gb=P) == abi.ERR_UNSUPPORTED  # prepared inputs carry one decay per head
    assert scan(abi, d, a=P + 4, alog=P, dtb=P) == abi.ERR_ALIGN  # the [N, H, K] decays load as vectors
    chunk = scan_desc(abi, flags=pk, qkv_dtype=1, gate_dtype=1, K=64, V=64, path=3)
    assert scan(abi, chunk, a=P, alog=P, dtb=P) == abi.ERR_UNSUPPORTED
    assert scan_capture(abi, scan_desc(abi, flags=pk, path=2)) == abi.ERR_UNSUPPORTED
    assert decode_step(abi, None, dict(flags=pk)) == abi.ERR_UNSUPPORTED
    n = ctypes.c_size_t(1)
    big = scan_desc(abi, flags=pk, qkv_dtype=1, gate_dtype=1, K=64, V=64, N=64 * 2)
    assert L.gdn_scan_workspace_bytes(ctypes.byref(big), ctypes.byref(n)) == abi.OK and n.value == 0


def scan_strided(abi, d, q=P, k=P, v=P, qs=None, ks=None, vs=None, qk=None, gb=None, off=P, out=P):
    w_qk, w_v = d.HQ * d.K, d.H * d.V
    s = abi.QKVStreams(q, k, v, w_qk if qs is None else qs, w_qk if ks is None else ks, w_v if vs is None else vs)
    return abi.lib().gdn_scan_varlen_strided(ctypes.byref(d), ctypes.byref(s), qk, gb, None, None, None, None, None,
                                             out, None, off, None, 0, None, None, None)


@pytest.mark.parametrize(
    "fields,kw,want",
    [
        ({}, dict(qs=63), "ERR_SHAPE"),  # q rows overlap (stride below the row width 2*32)
        ({}, dict(vs=60), "ERR_SHAPE"),
        ({}, dict(ks=65), "ERR_ALIGN"),  # rows would not start 16-byte aligned
        ({}, dict(v=P + 4), "ERR_ALIGN"),
        ({}, dict(q=None), "ERR_NULL"),
        ({}, dict(v=None), "ERR_NULL"),
        ({}, dict(qk=P, gb=P, q=None, k=None, qs=1, ks=1, off=None), "ERR_NULL"),  # prepared: q, k unread
        (dict(qkv_dtype=1, gate_dtype=1, V=33, H=2), dict(vs=72), "ERR_OK"),  # a packed row could not hold these
        (dict(N=2**30), dict(qs=2**40), "ERR_OVERFLOW"),
        ({}, dict(off=None), "ERR_NULL"),
    ],
)
def test_scan_strided_host_validation(abi, fields, kw, want):
    d = scan_desc(abi, **fields)
    if want == "ERR_OK":
        # valid streams: the call gets past the stream checks and fails on the missing offsets
        assert scan_strided(abi, d, off=None, **kw) == abi.ERR_NULL
        return
    assert scan_strided(abi, d, **kw) == getattr(abi, want)


def test_prepare_strided_host_validation(abi):
    L = abi.lib()
    d = scan_desc(abi)
    good = abi.QKVStreams(P, P, None, 64, 64, 0)  # v is not read by prepare
    assert L.gdn_prepare_qk_gates_strided(ctypes.byref(d), None, None, None, None, None, P, P, None) == abi.ERR_NULL
    bad = abi.QKVStreams(P, P, None, 62, 64, 0)
    assert L.gdn_prepare_qk_gates_strided(ctypes.byref(d), ctypes.byref(bad), None, None, None, None, P, P,
                                          None) == abi.ERR_SHAPE
    assert L.gdn_prepare_qk_gates_strided(ctypes.byref(d), ctypes.byref(good), None, None, None, None, None, None,
                                          None) == abi.ERR_NULL
    assert L.gdn_prepare_qk_gates_strided(ctypes.byref(d), ctypes.byref(good), None, None, None, None, P + 4, P,
                                          None) == abi.ERR_ALIGN


@pytest.mark.parametrize(
    "fields,kw,want",
    [
        (dict(B=0), {}, "ERR_SHAPE"),
        (dict(K=300), {}, "ERR_SHAPE"),
        (dict(path=3), {}, "ERR_UNSUPPORTED"),  # chunked path not eligible (fp32 I/O)
        ({}, dict(qkv=None), "ERR_NULL"),
        ({}, dict(off=None), "ERR_NULL"),
        ({}, dict(out=P + 2), "ERR_ALIGN"),
        # a chunked call whose workspace exceeds the library's device array
        (dict(B=1, N=1 << 16, HQ=32, H=32, K=128, V=128, qkv_dtype=1, gate_dtype=1, path=3), dict(a=P, alog=P, dtb=P),
         "ERR_WORKSPACE"),
    ],
)
def test_scan_noalloc_host_validation(abi, fields, kw, want):
    """gdn_scan_varlen_noalloc rejects these before it touches the device (no HIP call here)."""
    d = scan_desc(abi, **fields)
    a = dict(qkv=P, out=P, off=P, a=None, alog=None, dtb=None)
    a.update(kw)
    st = abi.lib().gdn_scan_varlen_noalloc(ctypes.byref(d), a["qkv"], None, None, a["a"], None, a["alog"], a["dtb"],
                                           None, a["out"], None, a["off"], None, None, None)
    assert st == getattr(abi, want)
