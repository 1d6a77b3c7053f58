"""GPU tests of gdn_decode_step (the conv and the recurrence of a decode step in one launch),
through the C ABI.

* Bit-identity with the two-call chain gdn_conv1d_varlen -> gdn_scan_varlen(DECODE) on the same
  inputs: outputs, final state and new conv window, in and out of place, over dtypes, key widths,
  GQA ratios, conv widths and dilations, with empty sequences, with and without bias, SiLU, initial
  states and gates.
* Parity with the oracle: oracle conv, its output rounded to the I/O type (the boundary between the
  two calls), oracle scan; the new window bit-exact.
* The decode-step contract: malformed offsets and sequences of more than one token write nothing
  and report their status."""
import numpy as np
import pytest

import cases
import oracle
import workloads
from gpu_util import CHAIN_STATE_TOL, SEQ_STATE_TOL, TOL, assert_close, bits, dev, dev_i32, ensure_built, f64, require_gpu, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def inputs(w):
    return dict(x=dev(w.x, w.io), cw=dev(w.conv_w, w.io), cb=dev(w.conv_bias, w.io),
                cst=dev(w.conv_state, w.conv_state_dtype), a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype),
                A_log=dev(w.A_log, "f32"), dtb=dev(w.dt_bias, "f32"), st=dev(w.state, "f32"),
                off=dev_i32(w.offsets))


def run_chain(torch, w, inplace=False):
    """gdn_conv1d_varlen then gdn_scan_varlen on the DECODE path."""
    import gated_delta_rule_varlen_amd as gdn

    t = inputs(w)
    cst_out = t["cst"] if (inplace and t["cst"] is not None) else (
        sentinel((w.B, w.C, w.L), w.conv_state_dtype) if w.L > 0 else None)
    y, cst_out = gdn.conv1d_varlen(t["x"], t["cw"], t["off"], bias=t["cb"], state_in=t["cst"], dilation=w.D,
                                   silu=w.silu, state_dtype=getattr(torch, {"f32": "float32", "bf16": "bfloat16",
                                                                             "f16": "float16"}[w.conv_state_dtype]),
                                   state_out=cst_out, write_state=w.L > 0)
    st_out = t["st"] if (inplace and t["st"] is not None) else sentinel((w.B, w.H, w.V, w.K), "f32")
    out, st_out, used = gdn.scan_varlen(y, t["off"], HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=t["a"], b=t["b"],
                                        A_log=t["A_log"], dt_bias=t["dtb"], state_in=t["st"], l2norm=w.l2norm,
                                        softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale, path="decode",
                                        out=sentinel((w.N, w.H, w.V), w.io), state_out=st_out)
    assert used == "decode"
    torch.cuda.synchronize()
    return out, st_out, cst_out


def run_fused(torch, w, inplace=False, offsets=None, dev_status=None):
    import gated_delta_rule_varlen_amd as gdn

    t = inputs(w)
    if offsets is not None:
        t["off"] = dev_i32(offsets)
    cdt = getattr(torch, {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}[w.conv_state_dtype])
    cst_out = t["cst"] if (inplace and t["cst"] is not None) else (
        sentinel((w.B, w.C, w.L), w.conv_state_dtype) if w.L > 0 else None)
    st_out = t["st"] if (inplace and t["st"] is not None) else sentinel((w.B, w.H, w.V, w.K), "f32")
    out, st_out, cst_out = gdn.decode_step(t["x"], t["cw"], t["off"], HQ=w.HQ, H=w.H, K=w.K, V=w.V, bias=t["cb"],
                                           conv_state_in=t["cst"], conv_state_out=cst_out, dilation=w.D,
                                           silu=w.silu, conv_state_dtype=cdt, a=t["a"], b=t["b"],
                                           A_log=t["A_log"], dt_bias=t["dtb"], state_in=t["st"], state_out=st_out,
                                           l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale,
                                           out=sentinel((w.N, w.H, w.V), w.io), write_state=w.L > 0,
                                           dev_status=dev_status)
    torch.cuda.synchronize()
    return out, st_out, cst_out


def small(name, seed, *, lengths, HQ, H, K, V, io="bf16", W=4, D=1, **kw):
    kw.setdefault("conv_state_dtype", "f32")
    return workloads.make(name=name, seed=seed, lengths=lengths, HQ=HQ, H=H, K=K, V=V, W=W, D=D, io=io, **kw)


LENS = [1, 0, 1, 1, 0, 1, 1, 1, 0, 1, 1, 1, 1, 0, 0, 1]  # empty sequences first, inside and last

CASES = {
    "bf16_k128_g2": dict(lengths=LENS, HQ=2, H=4, K=128, V=128),
    "bf16_k64_g1_bf16win": dict(lengths=LENS, HQ=2, H=2, K=64, V=64, conv_state_dtype="bf16"),
    "f16_k256_g4_v64": dict(lengths=LENS, HQ=1, H=4, K=256, V=64, io="f16"),
    "f32_k32_w2": dict(lengths=LENS, HQ=2, H=2, K=32, V=32, io="f32", W=2),
    "f16_k128_w3_d2_raw_gates": dict(lengths=LENS, HQ=2, H=4, K=128, V=32, io="f16", W=3, D=2, softplus=False,
                                     sigmoid=False, l2norm=False, decay_range=(-1.0, 0.0), beta_range=(0.0, 1.0),
                                     unit_k_scan=False, has_bias=False, silu=False),
    "bf16_w5_no_states": dict(lengths=LENS, HQ=2, H=4, K=64, V=64, W=5, conv_state_std=None, state_std=None),
    "bf16_w1_no_gates": dict(lengths=LENS, HQ=1, H=2, K=128, V=128, W=1, has_decay=False, has_beta=False),
    "bf16_v4_tail": dict(lengths=LENS, HQ=1, H=2, K=32, V=4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_is_bit_identical_to_the_two_call_chain(torch, name):
    w = small(name, 300 + sorted(CASES).index(name), **CASES[name])
    print(f"[decode_step] {name} B={w.B} N={w.N}", flush=True)
    o2, s2, c2 = run_chain(torch, w)
    o1, s1, c1 = run_fused(torch, w)
    assert np.array_equal(bits(o1), bits(o2)), "out"
    assert np.array_equal(bits(s1), bits(s2)), "state"
    if w.L > 0:
        assert np.array_equal(bits(c1), bits(c2)), "conv window"
    assert c1 is None or w.L > 0


@pytest.mark.parametrize("name", ["bf16_k128_g2", "f16_k256_g4_v64"])
def test_in_place_matches_out_of_place(torch, name):
    w = small(name, 300 + sorted(CASES).index(name), **CASES[name])
    o1, s1, c1 = run_fused(torch, w)
    o2, s2, c2 = run_fused(torch, w, inplace=True)
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(bits(s1), bits(s2))
    assert np.array_equal(bits(c1), bits(c2))


def oracle_chain(w):
    """Oracle conv, its output rounded to the I/O type (round to nearest even), oracle scan."""
    y, cwin = oracle.conv(w.x, w.conv_w, w.offsets, W=w.W, D=w.D, x_dtype=w.io, bias=w.conv_bias,
                          state_in=w.conv_state, state_dtype=w.conv_state_dtype, silu=w.silu)
    y_raw = workloads.to_raw(y.astype(np.float32), w.io)
    out, st = oracle.scan(y_raw, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                          a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state, l2norm=w.l2norm,
                          softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale)
    return out, st, cwin


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_matches_oracle(torch, name):
    w = small(name, 300 + sorted(CASES).index(name), **CASES[name])
    o, s, c = run_fused(torch, w)
    o_ref, s_ref, c_ref = oracle_chain(w)
    tol = TOL[w.io]
    e1 = assert_close(f64(o), o_ref, tol, "out")
    e2 = assert_close(f64(s), s_ref, CHAIN_STATE_TOL, "state")
    if w.L > 0:
        assert np.array_equal(f64(c), c_ref), "the new window is a copy: exact against the oracle's"
    print(f"  {name}: out {e1:.2e} state {e2:.2e}", flush=True)


def test_decode_workload_full_size(torch):
    """The benchmark's decode step (B=256, HQ=16, H=32, K=V=128, bf16, fp32 window and state), in
    place as the benchmark runs it: identical to the two-call chain; sampled heads against the oracle."""
    w = cases.get("decode")
    o2, s2, c2 = run_chain(torch, w)
    o1, s1, c1 = run_fused(torch, w, inplace=True)
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(bits(s1), bits(s2))
    assert np.array_equal(bits(c1), bits(c2))
    # oracle on the first 32 sequences (every head)
    nb = 32
    sub = workloads.Workload(**{**w.__dict__, "B": nb, "N": nb, "offsets": w.offsets[:nb + 1], "x": w.x[:nb],
                                "qkv": w.qkv[:nb], "a": w.a[:nb], "b": w.b[:nb], "conv_state": w.conv_state[:nb],
                                "state": w.state[:nb]})
    o_ref, s_ref, _ = oracle_chain(sub)
    assert_close(f64(o1)[:nb], o_ref, TOL[w.io], "out")
    assert_close(f64(s1)[:nb], s_ref, CHAIN_STATE_TOL, "state")


@pytest.mark.parametrize("state_inplace", [False, True])
def test_decode_workload_full_size_separate_window(torch, state_inplace):
    """The benchmark's decode step with the new window in a separate buffer (the column-tile form of
    large batches; the state updated in place or not): identical to the two-call chain, bit for bit,
    and sampled sequences against the oracle."""
    import gated_delta_rule_varlen_amd as gdn

    w = cases.get("decode")
    o2, s2, c2 = run_chain(torch, w)
    t = inputs(w)
    cst_out = sentinel((w.B, w.C, w.L), w.conv_state_dtype)
    st_out = t["st"] if state_inplace else sentinel((w.B, w.H, w.V, w.K), "f32")
    o1, s1, c1 = gdn.decode_step(t["x"], t["cw"], t["off"], HQ=w.HQ, H=w.H, K=w.K, V=w.V, bias=t["cb"],
                                 conv_state_in=t["cst"], conv_state_out=cst_out, dilation=w.D, silu=w.silu,
                                 conv_state_dtype=torch.float32, a=t["a"], b=t["b"], A_log=t["A_log"],
                                 dt_bias=t["dtb"], state_in=t["st"], state_out=st_out, l2norm=w.l2norm,
                                 softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale,
                                 out=sentinel((w.N, w.H, w.V), w.io))
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(bits(s1), bits(s2))
    assert np.array_equal(bits(c1), bits(c2))


def test_malformed_offsets_and_long_sequences_write_nothing(torch):
    w = small("contract", 399, lengths=[1, 1, 0, 1], HQ=1, H=2, K=64, V=64)
    import gated_delta_rule_varlen_amd as gdn  # noqa: F401

    for case, off, want in [("first != 0", [1, 1, 2, 2, 4], -9), ("decreasing", [0, 2, 1, 3, 3], -9),
                            ("last != N", [0, 1, 2, 2, 4], -9), ("two tokens", [0, 2, 2, 2, 3], -6)]:
        if case == "two tokens":
            w2 = small("contract2", 398, lengths=[2, 0, 0, 1], HQ=1, H=2, K=64, V=64)
        else:
            w2 = w
        status = dev_i32(np.array([12345]))
        o, s, c = run_fused(torch, w2, offsets=np.array(off, np.int32), dev_status=status)
        assert int(status.cpu()[0]) == want, case
        assert np.all(bits(o) == bits(sentinel(tuple(o.shape), w2.io))), case
        assert np.all(bits(s) == bits(sentinel(tuple(s.shape), "f32"))), case
        assert np.all(bits(c) == bits(sentinel(tuple(c.shape), w2.conv_state_dtype))), case
    status = dev_i32(np.array([12345]))
    run_fused(torch, w, dev_status=status)
    assert int(status.cpu()[0]) == 0
