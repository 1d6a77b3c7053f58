"""GPU tests of the separate-token-stream entry points (gdn_scan_varlen_strided,
gdn_prepare_qk_gates_strided) through the C ABI.

* Views of a packed [q | k | v] buffer (row stride C), separate contiguous buffers and separate
  buffers with padded rows all give results bit-identical to the packed entry points, on the
  DECODE, SEQ and CHUNK paths, with fused and prepared inputs.
* A value width no packed 16-byte-aligned row can hold (bf16, H*V odd) runs through the strided
  streams and matches the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import SEQ_STATE_TOL, TOL, assert_close, bits, dev, dev_i32, ensure_built, f64, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def layouts(torch, w):
    """(name, q, k, v) device views of the workload's token rows in three layouts."""
    qkv = dev(w.qkv, w.io)
    HQK, HV = w.HQ * w.K, w.H * w.V
    views = qkv[:, :HQK], qkv[:, HQK:2 * HQK], qkv[:, 2 * HQK:]
    yield "packed_views", views[0].view(w.N, w.HQ, w.K), views[1], views[2].view(w.N, w.H, w.V)
    yield "separate", *(t.contiguous() for t in views)
    padded = []
    for t, pad in zip(views, (32, 64, 8)):
        buf = torch.zeros((w.N, t.shape[1] + pad), dtype=t.dtype, device="cuda")
        buf[:, :t.shape[1]] = t
        padded.append(buf[:, :t.shape[1]])
    yield "padded", *padded


def scan_kw(w, torch):
    return dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype),
                A_log=dev(w.A_log, "f32"), dt_bias=dev(w.dt_bias, "f32"), state_in=dev(w.state, "f32"),
                l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale)


CASES = [
    ("decode", dict(lengths=[1, 0, 1, 3, 1, 2], HQ=2, H=4, K=128, V=128, io="bf16")),
    ("seq", dict(lengths=[37, 0, 5, 64, 1], HQ=2, H=4, K=64, V=64, io="f32")),
    ("seq", dict(lengths=[20, 9], HQ=1, H=2, K=256, V=32, io="f16")),
    ("chunk", dict(lengths=[150, 70, 0, 129], HQ=2, H=4, K=128, V=128, io="bf16")),
    ("chunk", dict(lengths=[100, 64], HQ=1, H=2, K=64, V=64, io="f16")),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("prepared", [False, True])
def test_strided_streams_are_bit_identical_to_packed(torch, case, prepared):
    import gated_delta_rule_varlen_amd as gdn

    path, kw = CASES[case]
    if prepared and path == "chunk":
        pytest.skip("the chunked form takes fused inputs only")
    w = workloads.make(name=f"strided_{case}", seed=700 + case, **kw)
    common = scan_kw(w, torch)
    off = dev_i32(w.offsets)
    qkv = dev(w.qkv, w.io)
    qk = gb = None
    if prepared:
        qk, gb = gdn.prepare_qk_gates(qkv, HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=common["a"], b=common["b"],
                                      A_log=common["A_log"], dt_bias=common["dt_bias"], l2norm=w.l2norm,
                                      softplus=w.softplus, sigmoid=w.sigmoid)
    o_ref, s_ref, used = gdn.scan_varlen(qkv, off, path=path, qk_prep=qk, gb_prep=gb, **common)
    assert used == path
    for name, q, k, v in layouts(torch, w):
        print(f"[strided] {path} case {case} prepared={prepared} {name}", flush=True)
        if prepared:
            qk2, gb2 = gdn.prepare_qk_gates_strided(q, k, HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=common["a"],
                                                    b=common["b"], A_log=common["A_log"],
                                                    dt_bias=common["dt_bias"], l2norm=w.l2norm, softplus=w.softplus,
                                                    sigmoid=w.sigmoid)
            torch.cuda.synchronize()
            assert np.array_equal(bits(qk2), bits(qk)) and np.array_equal(bits(gb2), bits(gb)), name
            q = k = None  # prepared scans read only v from the streams
        o, s, used = gdn.scan_varlen_strided(q, k, v, off, path=path, qk_prep=qk, gb_prep=gb, **common)
        torch.cuda.synchronize()
        assert used == path
        assert np.array_equal(bits(o), bits(o_ref)), name
        assert np.array_equal(bits(s), bits(s_ref)), name


@pytest.mark.parametrize("path", ["decode", "seq"])
def test_strided_unpackable_value_width_matches_oracle(torch, path):
    """bf16 with H*V = 66: a packed row (2*HQ*K + 66 elements) would not start 16-byte aligned."""
    import gated_delta_rule_varlen_amd as gdn

    w = workloads.make(name="strided_v33", seed=720, lengths=[12, 1, 0, 30], HQ=1, H=2, K=64, V=33, io="bf16")
    HQK, HV = w.HQ * w.K, w.H * w.V
    raw = np.ascontiguousarray(w.qkv)
    q = dev(np.ascontiguousarray(raw[:, :HQK]), w.io)
    k = dev(np.ascontiguousarray(raw[:, HQK:2 * HQK]), w.io)
    vbuf = dev(np.ascontiguousarray(np.pad(raw[:, 2 * HQK:], ((0, 0), (0, 72 - HV)))), w.io)  # rows of 144 bytes
    out, st, used = gdn.scan_varlen_strided(q, k, vbuf[:, :HV], dev_i32(w.offsets), path=path, **scan_kw(w, torch))
    torch.cuda.synchronize()
    assert used == path
    o_ref, s_ref = oracle.scan(raw, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                               a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state, l2norm=w.l2norm,
                               softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale)
    e1 = assert_close(f64(out), o_ref, TOL[w.io], "out")
    e2 = assert_close(f64(st), s_ref, SEQ_STATE_TOL, "state")
    print(f"  v33 {path}: out {e1:.2e} state {e2:.2e}", flush=True)
