"""GPU parity at key widths other than 32, 64, 128 and 256, through the C ABI.

The pages define the recurrence for every K <= 256.  Widths other than the compiled ones run on the
next compiled width with the elements past K zero; these tests hold DECODE and SEQ (fused and
prepared inputs), the prepare pass and the capture capsule to the oracle at K = 48, 96 and 192 and
at widths that are not multiples of 8 or 4 (K = 20, 50, 7, 200), with ragged sequences (empty,
single-token, short and multi-chunk ones) and GQA.  Outputs at the I/O tolerance, the fp32 final
state at the token-sequential bound; empty sequences keep their state bit for bit."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (PREP_TOL, SEQ_STATE_TOL, TOL, assert_close, assert_close_slices, bits, dev, dev_i32,
                      ensure_built, f64, require_gpu)
from test_gpu_scan import gpu_scan

pytestmark = pytest.mark.gpu

# packed rows stay a multiple of 16 bytes: C = 2 HQ K + H V elements
WIDTHS = {
    "k48_bf16_g2": dict(HQ=2, H=4, K=48, V=64, io="bf16"),
    "k96_f16": dict(HQ=1, H=2, K=96, V=64, io="f16"),
    "k192_bf16": dict(HQ=2, H=2, K=192, V=32, io="bf16"),
    "k20_bf16_g2": dict(HQ=2, H=4, K=20, V=8, io="bf16"),
    "k50_f32_v14": dict(HQ=1, H=2, K=50, V=14, io="f32"),
    "k7_f32": dict(HQ=1, H=1, K=7, V=2, io="f32"),
    "k200_f16_v24": dict(HQ=1, H=1, K=200, V=24, io="f16"),
}
LENS = [0, 1, 5, 40, 130, 3]


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def workload(name):
    return workloads.make(name=name, seed=900 + sorted(WIDTHS).index(name), lengths=LENS, conv_state_dtype="f32",
                          **WIDTHS[name])


@pytest.mark.parametrize("mode", ["fused", "prepared"])
@pytest.mark.parametrize("path", ["decode", "seq"])
@pytest.mark.parametrize("name", sorted(WIDTHS))
def test_key_width_against_oracle(torch, name, path, mode):
    w = workload(name)
    print(f"[key width] {name} path={path} mode={mode} K={w.K} V={w.V} {w.io}", flush=True)
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                               gate_dtype=w.gate_dtype, a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias,
                               state_in=w.state)
    out, st, used = gpu_scan(torch, w, path, mode == "prepared")
    assert used == path
    assert_close(f64(out), o_ref, TOL[w.io], f"{name} {path} {mode} out")
    assert_close_slices(f64(out), o_ref, w.lengths, TOL[w.io], f"{name} {path} {mode} out")
    assert_close(f64(st), s_ref, SEQ_STATE_TOL, f"{name} {path} {mode} state")
    empty = np.flatnonzero(w.lengths == 0)
    assert np.array_equal(bits(st)[empty], w.state[empty].view(np.int32))


@pytest.mark.parametrize("name", sorted(WIDTHS))
def test_key_width_prepare_against_oracle(torch, name):
    import gated_delta_rule_varlen_amd as gdn

    w = workload(name)
    qk, gb = gdn.prepare_qk_gates(dev(w.qkv, w.io), HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=dev(w.a, w.gate_dtype),
                                  b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"), dt_bias=dev(w.dt_bias, "f32"),
                                  l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid)
    torch.cuda.synchronize()
    qk_ref, gb_ref = oracle.prepare(w.qkv, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                                    a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, l2norm=w.l2norm,
                                    softplus=w.softplus, sigmoid=w.sigmoid)
    assert tuple(qk.shape) == (2, w.N, w.HQ, w.K)
    for plane, nm in enumerate("qk"):
        assert_close(f64(qk)[plane], qk_ref[plane], PREP_TOL, f"{name} prepare {nm}-hat")
    assert_close(f64(gb), gb_ref, PREP_TOL, f"{name} prepare gates")


@pytest.mark.parametrize("path", ["decode", "seq"])
def test_key_width_capture_against_oracle(torch, path):
    """The capsule's k^ rows are K wide at a padded width too."""
    import gated_delta_rule_varlen_amd as gdn

    w = workload("k48_bf16_g2")
    cap = 4
    counts = np.array([2, 1, 4, 3, 9, 0], np.int32)
    _, _, caps, used = gdn.scan_varlen_capture(dev(w.qkv, w.io), dev_i32(w.offsets), cap=cap, counts=dev_i32(counts),
                                               HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=dev(w.a, w.gate_dtype),
                                               b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"),
                                               dt_bias=dev(w.dt_bias, "f32"), state_in=dev(w.state, "f32"), path=path)
    torch.cuda.synchronize()
    assert used == path
    _, _, ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                            a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state, counts=counts, cap=cap)
    got = f64(caps)
    assert np.all(got[ref == 0] == 0)
    assert_close(got, ref, TOL[w.io], f"k48 capture {path}")


def test_key_width_decode_batch_of_single_tokens(torch):
    """The single-token streaming form and the short-sequence form at a padded width."""
    w = workloads.make(name="k96_decode", seed=950, lengths=[1] * 40 + [0, 3, 7, 1], HQ=2, H=4, K=96, V=64,
                       io="bf16", conv_state_dtype="f32")
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                               gate_dtype=w.gate_dtype, a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias,
                               state_in=w.state)
    for lens in (w.lengths,):
        out, st, used = gpu_scan(torch, w, "decode", False)
        assert used == "decode"
        assert_close(f64(out), o_ref, TOL[w.io], "k96 decode out")
        assert_close(f64(st), s_ref, SEQ_STATE_TOL, "k96 decode state")
    w1 = workloads.make(name="k96_step", seed=951, lengths=[1] * 64, HQ=2, H=4, K=96, V=64, io="bf16",
                        conv_state_dtype="f32")
    o_ref, s_ref = oracle.scan(w1.qkv, w1.offsets, HQ=w1.HQ, H=w1.H, K=w1.K, V=w1.V, qkv_dtype=w1.io,
                               gate_dtype=w1.gate_dtype, a=w1.a, b=w1.b, A_log=w1.A_log, dt_bias=w1.dt_bias,
                               state_in=w1.state)
    out, st, used = gpu_scan(torch, w1, "decode", False)
    assert used == "decode"
    assert_close(f64(out), o_ref, TOL[w1.io], "k96 step out")
    assert_close(f64(st), s_ref, SEQ_STATE_TOL, "k96 step state")
