"""GPU parity of the per-key-channel decay (GDN_GATE_PER_KEY: a [N, H, K] decay input, the
gate_per_channel form of the GatedDeltaNet thunk on the rlx-cpu thunk/types.rs page) through the
C ABI, against the oracle on the same inputs: DECODE (the single-token streaming form too) and SEQ
(all three SEQ tile shapes), fp32 / bf16 / fp16 I/O with fp32 or I/O-typed decay inputs, softplus
and raw log-decays, with and without the retrieval term, GQA, and every instantiated key width."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import SEQ_STATE_TOL, TOL, assert_close, dev, dev_i32, ensure_built, f64, require_gpu, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def per_key_problem(name, seed, lengths, HQ, H, K, V, io, *, softplus=True, gate_dtype=None, **kw):
    w = workloads.make(name=name, seed=seed, lengths=lengths, HQ=HQ, H=H, K=K, V=V, io=io, softplus=softplus,
                       gate_dtype=gate_dtype, **kw)
    rng = np.random.default_rng(seed + 1000)
    a = rng.standard_normal((w.N, H, K)).astype(np.float32) if softplus else \
        rng.uniform(-1.0, 0.0, (w.N, H, K)).astype(np.float32)
    return w, workloads.to_raw(a, w.gate_dtype)


def run(torch, w, a_pk, path, retrieve=True):
    import gated_delta_rule_varlen_amd as gdn

    out, st, used = gdn.scan_varlen(dev(w.qkv, w.io), dev_i32(w.offsets), HQ=w.HQ, H=w.H, K=w.K, V=w.V,
                                    a=dev(a_pk, w.gate_dtype), b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"),
                                    dt_bias=dev(w.dt_bias, "f32"), state_in=dev(w.state, "f32"), l2norm=w.l2norm,
                                    softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale, path=path,
                                    retrieve=retrieve, gate_per_key=True, out=sentinel((w.N, w.H, w.V), w.io),
                                    state_out=sentinel((w.B, w.H, w.V, w.K), "f32"))
    torch.cuda.synchronize()
    assert used == path
    return out, st


def check(w, a_pk, out, st, retrieve=True, what=""):
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                               gate_dtype=w.gate_dtype, a=a_pk, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias,
                               state_in=w.state, l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid,
                               scale=w.scale, retrieve=retrieve, gate_per_key=True)
    tol = TOL[w.io]
    e1 = assert_close(f64(out), o_ref, tol, f"{what} out")
    e2 = assert_close(f64(st), s_ref, SEQ_STATE_TOL, f"{what} state")
    print(f"  {what}: out {e1:.2e} state {e2:.2e}", flush=True)


LENS = [9, 0, 1, 17, 4, 33, 1, 2]
CASES = {
    "f32_k32_g2": dict(HQ=2, H=4, K=32, V=32, io="f32"),
    "f32_k64_raw": dict(HQ=1, H=2, K=64, V=48, io="f32", softplus=False),
    "bf16_k128_f32gates": dict(HQ=2, H=4, K=128, V=128, io="bf16", gate_dtype="f32"),
    "f16_k256_v64": dict(HQ=1, H=2, K=256, V=64, io="f16"),
    "bf16_k64_bf16gates_g4": dict(HQ=1, H=4, K=64, V=64, io="bf16"),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("path", ["decode", "seq"])
def test_per_key_gate_matches_oracle(torch, name, path):
    w, a_pk = per_key_problem(name, 600 + sorted(CASES).index(name), LENS, **CASES[name])
    print(f"[per-key] {name} {path}", flush=True)
    out, st = run(torch, w, a_pk, path)
    check(w, a_pk, out, st, what=f"{name}/{path}")


@pytest.mark.parametrize("path", ["decode", "seq"])
def test_per_key_gate_without_retrieval(torch, path):
    w, a_pk = per_key_problem("pk_gated", 620, LENS, HQ=2, H=4, K=64, V=64, io="f32")
    out, st = run(torch, w, a_pk, path, retrieve=False)
    check(w, a_pk, out, st, retrieve=False, what=f"gated/{path}")


def test_per_key_gate_single_token_streaming(torch):
    """Decode-step shape: one token per sequence, carried state, whole column tiles."""
    w, a_pk = per_key_problem("pk_stream", 621, [1] * 16 + [0, 1], HQ=2, H=4, K=128, V=128, io="bf16")
    out, st = run(torch, w, a_pk, "decode")
    check(w, a_pk, out, st, what="stream")


def test_per_key_gate_wide_seq_tile(torch):
    """Enough columns for the two-columns-per-group SEQ tile (B*H*V/128 >= 1024)."""
    w, a_pk = per_key_problem("pk_wide", 622, [6, 3, 0, 9] * 16, HQ=4, H=16, K=64, V=128, io="bf16",
                              gate_dtype="f32")
    out, st = run(torch, w, a_pk, "seq")
    check(w, a_pk, out, st, what="wide seq")


def test_auto_never_takes_chunk_with_per_key_gate(torch):
    w, a_pk = per_key_problem("pk_auto", 623, [160, 130], HQ=1, H=2, K=64, V=64, io="bf16")
    import gated_delta_rule_varlen_amd as gdn

    _, _, used = gdn.scan_varlen(dev(w.qkv, w.io), dev_i32(w.offsets), HQ=w.HQ, H=w.H, K=w.K, V=w.V,
                                 a=dev(a_pk, w.gate_dtype), b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"),
                                 dt_bias=dev(w.dt_bias, "f32"), gate_per_key=True)
    torch.cuda.synchronize()
    assert used == "seq"


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_per_key_gate_short_sequences(torch, io):
    """Verification-step shape (2..8 tokens per sequence): the DECODE path's short-sequence form with
    decays staged per key channel."""
    w, a_pk = per_key_problem(f"pk_short_{io}", 624, [5, 2, 8, 3, 5, 7, 1, 0, 4, 6], HQ=2, H=4, K=128, V=64, io=io)
    out, st = run(torch, w, a_pk, "decode")
    check(w, a_pk, out, st, what=f"short {io}")
