"""ctypes view of libgdn's C ABI (include/gdn.h).  Loading fails loudly when the library is absent."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

# gdn_status
OK = 0
ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_OVERFLOW, ERR_ALIGN = -1, -2, -3, -4, -5
ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_OFFSETS = -6, -7, -8, -9
# the device array gdn_scan_varlen_noalloc uses as its workspace (GDN_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20
# gdn_dtype
F32, BF16, F16 = 0, 1, 2
# flags
CONV_SILU = 1
L2NORM, SOFTPLUS, SIGMOID, NO_RETRIEVE, GATE_PER_KEY = 1, 2, 4, 8, 16
# gdn_path
PATH_AUTO, PATH_DECODE, PATH_SEQ, PATH_CHUNK = 0, 1, 2, 3
PATH_NAMES = {PATH_AUTO: "auto", PATH_DECODE: "decode", PATH_SEQ: "seq", PATH_CHUNK: "chunk"}
PATH_CODES = {v: k for k, v in PATH_NAMES.items()}

# Every symbol include/gdn.h declares.
EXPORTS = (
    "gdn_conv1d_varlen",
    "gdn_conv1d_varlen_capture",
    "gdn_prepare_qk_gates",
    "gdn_prepare_qk_gates_strided",
    "gdn_scan_varlen",
    "gdn_scan_varlen_capture",
    "gdn_scan_varlen_strided",
    "gdn_scan_varlen_noalloc",
    "gdn_scan_workspace_bytes",
    "gdn_decode_step",
    "gdn_status_string",
    "gdn_abi_version",
)


class ConvDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("C", ctypes.c_int32),
        ("W", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("x_dtype", ctypes.c_int32),
        ("state_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class ScanDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("HQ", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("V", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32),
        ("gate_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("scale", ctypes.c_float),
        ("path", ctypes.c_int32),
    ]


class QKVStreams(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64),
        ("k_stride", ctypes.c_int64),
        ("v_stride", ctypes.c_int64),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgdn.so.  Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_varlen_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p, st = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_int
        L.gdn_conv1d_varlen.argtypes = [ctypes.POINTER(ConvDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdn_conv1d_varlen.restype = st
        L.gdn_conv1d_varlen_capture.argtypes = [ctypes.POINTER(ConvDesc)] + [vp] * 7 + [ctypes.c_int32, vp, vp, vp, vp]
        L.gdn_conv1d_varlen_capture.restype = st
        L.gdn_prepare_qk_gates.argtypes = [ctypes.POINTER(ScanDesc), vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdn_prepare_qk_gates.restype = st
        L.gdn_prepare_qk_gates_strided.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(QKVStreams)] + [vp] * 7
        L.gdn_prepare_qk_gates_strided.restype = st
        L.gdn_scan_varlen.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 12 + [ctypes.c_size_t, vp, i32p, vp]
        L.gdn_scan_varlen.restype = st
        L.gdn_scan_varlen_capture.argtypes = ([ctypes.POINTER(ScanDesc)] + [vp] * 11 + [ctypes.c_int32, vp, vp, vp, vp,
                                              ctypes.c_size_t, vp, i32p, vp])
        L.gdn_scan_varlen_capture.restype = st
        L.gdn_scan_varlen_strided.argtypes = ([ctypes.POINTER(ScanDesc), ctypes.POINTER(QKVStreams)] + [vp] * 11 +
                                              [ctypes.c_size_t, vp, i32p, vp])
        L.gdn_scan_varlen_strided.restype = st
        L.gdn_scan_varlen_noalloc.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 11 + [vp, i32p, vp]
        L.gdn_scan_varlen_noalloc.restype = st
        L.gdn_decode_step.argtypes = [ctypes.POINTER(ConvDesc), ctypes.POINTER(ScanDesc)] + [vp] * 15
        L.gdn_decode_step.restype = st
        L.gdn_scan_workspace_bytes.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(ctypes.c_size_t)]
        L.gdn_scan_workspace_bytes.restype = st
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()
