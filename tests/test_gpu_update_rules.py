"""GPU parity of the update rules without the retrieval term (GDN_NO_RETRIEVE: the pages' "linear"
rule without a decay input and "gated" rule with one) through the C ABI, against the oracle on the
same inputs: DECODE and SEQ paths, fused and prepared inputs, and the single-launch decode step."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import SEQ_STATE_TOL, TOL, assert_close, bits, dev, dev_i32, ensure_built, f64, require_gpu, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def rule_workload(io, decay, seed):
    # ragged lengths with an empty sequence; q/k normalised in-kernel; raw log-decays in [-1, 0]
    return workloads.make(name=f"rule_{io}_{decay}", seed=seed, lengths=[37, 0, 5, 130, 1, 64], HQ=2, H=4, K=64,
                          V=32, io=io, softplus=False, decay_range=(-1.0, 0.0), has_decay=decay)


def oracle_ref(w):
    return oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                       a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state, l2norm=w.l2norm,
                       softplus=w.softplus, sigmoid=w.sigmoid, retrieve=False)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("decay", [False, True])
@pytest.mark.parametrize("path", ["decode", "seq"])
@pytest.mark.parametrize("prepared", [False, True])
def test_no_retrieval_matches_oracle(torch, io, decay, path, prepared):
    import gated_delta_rule_varlen_amd as gdn

    w = rule_workload(io, decay, 70 + 2 * decay + (io == "bf16"))
    qkv = dev(w.qkv, w.io)
    a, b = dev(w.a, w.gate_dtype), dev(w.b, w.gate_dtype)
    qk = gb = None
    if prepared:
        qk, gb = gdn.prepare_qk_gates(qkv, HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=a, b=b, l2norm=w.l2norm,
                                      softplus=w.softplus, sigmoid=w.sigmoid)
    out, st, used = gdn.scan_varlen(qkv, dev_i32(w.offsets), HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=a, b=b,
                                    state_in=dev(w.state, "f32"), qk_prep=qk, gb_prep=gb, l2norm=w.l2norm,
                                    softplus=w.softplus, sigmoid=w.sigmoid, path=path, retrieve=False,
                                    out=sentinel((w.N, w.H, w.V), w.io),
                                    state_out=sentinel((w.B, w.H, w.V, w.K), "f32"))
    torch.cuda.synchronize()
    assert used == path
    o_ref, s_ref = oracle_ref(w)
    tol = TOL[w.io]
    e1 = assert_close(f64(out), o_ref, tol, "out")
    e2 = assert_close(f64(st), s_ref, SEQ_STATE_TOL, "state")
    print(f"  {io} decay={decay} {path} prepared={prepared}: out {e1:.2e} state {e2:.2e}", flush=True)


def test_auto_path_never_takes_the_chunked_form_without_retrieval(torch):
    import gated_delta_rule_varlen_amd as gdn

    w = workloads.make(name="rule_prefill", seed=77, lengths=[300, 200], HQ=2, H=4, K=64, V=64, io="bf16")
    out, st, used = gdn.scan_varlen(dev(w.qkv, w.io), dev_i32(w.offsets), HQ=w.HQ, H=w.H, K=w.K, V=w.V,
                                    a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"),
                                    dt_bias=dev(w.dt_bias, "f32"), state_in=dev(w.state, "f32"), retrieve=False)
    torch.cuda.synchronize()
    assert used == "seq"
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, a=w.a, b=w.b,
                               A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state, retrieve=False)
    assert_close(f64(out), o_ref, TOL[w.io], "out")
    assert_close(f64(st), s_ref, TOL[w.io], "state")


def test_fused_decode_step_without_retrieval_matches_two_calls(torch):
    import gated_delta_rule_varlen_amd as gdn

    w = workloads.make(name="rule_decode", seed=78, lengths=[1, 0, 1, 1, 1, 0, 1, 1], HQ=2, H=4, K=128, V=128,
                       io="bf16", conv_state_dtype="f32")
    x, cw, cb = dev(w.x, w.io), dev(w.conv_w, w.io), dev(w.conv_bias, w.io)
    off = dev_i32(w.offsets)
    g = dict(a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"),
             dt_bias=dev(w.dt_bias, "f32"))
    y, c2 = gdn.conv1d_varlen(x, cw, off, bias=cb, state_in=dev(w.conv_state, "f32"), dilation=w.D, silu=w.silu)
    o2, s2, _ = gdn.scan_varlen(y, off, HQ=w.HQ, H=w.H, K=w.K, V=w.V, state_in=dev(w.state, "f32"), path="decode",
                                retrieve=False, **g)
    o1, s1, c1 = gdn.decode_step(x, cw, off, HQ=w.HQ, H=w.H, K=w.K, V=w.V, bias=cb,
                                 conv_state_in=dev(w.conv_state, "f32"), state_in=dev(w.state, "f32"),
                                 retrieve=False, **g)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(s1), bits(s2))
    assert np.array_equal(bits(c1), bits(c2))
