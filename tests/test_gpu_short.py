"""GPU parity of the DECODE path's short-sequence form (sequences of 2 to 8 tokens carried column by
column with token operands staged once per block) through the C ABI, against the oracle: every
instantiated key width, fp32 / bf16 / fp16 I/O, fused and prepared inputs, softplus and raw gates,
with and without the retrieval term, ragged batches that mix 0, 1, 2..8 and longer sequences (the
longer ones take the general loop of the same launch), whole and partial column tiles, and AUTO's
choice of DECODE for short batches."""
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


LENS = [2, 5, 0, 8, 1, 3, 7, 9, 4, 6, 2, 13]  # 9 and 13 take the general loop


def run(torch, w, *, path="decode", prepared=False, retrieve=True, inplace=False):
    import gated_delta_rule_varlen_amd as gdn

    qkv = dev(w.qkv, w.io)
    a, b = dev(w.a, w.gate_dtype), dev(w.b, w.gate_dtype)
    A_log, dtb = dev(w.A_log, "f32"), dev(w.dt_bias, "f32")
    qk = gb = None
    if prepared:
        qk, gb = gdn.prepare_qk_gates(qkv, HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=a, b=b, A_log=A_log, dt_bias=dtb,
                                      l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid)
    st_in = dev(w.state, "f32")
    st_out = st_in if inplace else sentinel((w.B, w.H, w.V, w.K), "f32")
    out, st, used = gdn.scan_varlen(qkv, dev_i32(w.offsets), HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=a, b=b, A_log=A_log,
                                    dt_bias=dtb, state_in=st_in, qk_prep=qk, gb_prep=gb, l2norm=w.l2norm,
                                    softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale, path=path,
                                    retrieve=retrieve, out=sentinel((w.N, w.H, w.V), w.io), state_out=st_out)
    torch.cuda.synchronize()
    return out, st, used


def check(w, out, st, retrieve=True, what=""):
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                               gate_dtype=w.gate_dtype, a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias,
                               state_in=w.state, l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid,
                               scale=w.scale, retrieve=retrieve)
    tol = TOL[w.io]
    e1 = assert_close(f64(out), o_ref, tol, f"{what} out")
    e2 = assert_close(f64(st), s_ref, SEQ_STATE_TOL, f"{what} state")
    print(f"  {what}: out {e1:.2e} state {e2:.2e}", flush=True)


CASES = {
    # whole column tiles (V a multiple of the block's columns: 128 at K=32, 64 at K=64/128, 32 at K=256)
    "f32_k32_v128": dict(HQ=2, H=2, K=32, V=128, io="f32"),
    "bf16_k64_g2": dict(HQ=2, H=4, K=64, V=64, io="bf16"),
    "bf16_k128_g2": dict(HQ=2, H=4, K=128, V=128, io="bf16"),
    "f16_k256_v32_g4": dict(HQ=1, H=4, K=256, V=32, io="f16"),
    "f32_k128_f32gates": dict(HQ=1, H=2, K=128, V=64, io="f32", gate_dtype="f32"),
    "bf16_k64_raw_gates": dict(HQ=2, H=2, K=64, V=64, io="bf16", softplus=False, sigmoid=False, l2norm=False,
                               decay_range=(-1.0, 0.0), beta_range=(0.0, 1.0), unit_k_scan=True),
    # a partial last tile: those blocks take the general loop
    "f32_k64_v96": dict(HQ=1, H=2, K=64, V=96, io="f32"),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("prepared", [False, True])
def test_short_sequences_match_oracle(torch, name, prepared):
    w = workloads.make(name=name, seed=800 + sorted(CASES).index(name), lengths=LENS, **CASES[name])
    print(f"[short] {name} prepared={prepared}", flush=True)
    out, st, used = run(torch, w, prepared=prepared)
    assert used == "decode"
    check(w, out, st, what=f"{name}/{prepared}")


@pytest.mark.parametrize("decay", [False, True])
def test_short_sequences_without_retrieval(torch, decay):
    w = workloads.make(name="short_rule", seed=820 + decay, lengths=LENS, HQ=2, H=4, K=128, V=64, io="f32",
                       has_decay=decay, softplus=False, decay_range=(-1.0, 0.0))
    out, st, _ = run(torch, w, retrieve=False)
    check(w, out, st, retrieve=False, what=f"no-retrieve decay={decay}")


def test_short_in_place_matches_out_of_place(torch):
    w = workloads.make(name="short_inplace", seed=830, lengths=LENS, HQ=2, H=4, K=128, V=128, io="bf16")
    o1, s1, _ = run(torch, w)
    o2, s2, _ = run(torch, w, inplace=True)
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(s1), bits(s2))


def test_auto_takes_decode_for_short_batches(torch):
    """Verification-step shape (every sequence 5 tokens): AUTO runs DECODE, which matches the oracle
    and the SEQ path on the same inputs."""
    w = workloads.make(name="short_auto", seed=831, lengths=[5] * 24, HQ=2, H=4, K=128, V=128, io="bf16")
    out, st, used = run(torch, w, path="auto")
    assert used == "decode"
    check(w, out, st, what="auto")
    o2, s2, used2 = run(torch, w, path="seq")
    assert used2 == "seq"
    assert_close(f64(out), f64(o2), TOL[w.io], "decode vs seq out")
    assert_close(f64(st), f64(s2), SEQ_STATE_TOL, "decode vs seq state")


def test_short_sequences_with_extreme_decays(torch):
    """Raw log-decays from -200 (a decay that is 0 in fp32) to +10 (growth) on some tokens: the scaled
    state of the short form folds its scale into the state whenever it leaves [1e-30, 1e30]."""
    w = workloads.make(name="short_extreme", seed=840, lengths=[8, 6, 8, 3, 5, 8], HQ=1, H=2, K=64, V=64, io="f32",
                       softplus=False, decay_range=(-1.0, 0.0))
    a = workloads.from_raw(w.a, w.gate_dtype).astype(np.float32).copy()
    rng = np.random.default_rng(841)
    idx = rng.choice(a.size, size=a.size // 4, replace=False)
    a.flat[idx] = rng.choice(np.array([-200.0, -80.0, -40.0, 4.0, 10.0], np.float32), size=idx.size)
    w.a = workloads.to_raw(a, w.gate_dtype)
    out, st, used = run(torch, w)
    assert used == "decode"
    assert np.all(np.isfinite(f64(out))) and np.all(np.isfinite(f64(st)))
    check(w, out, st, what="extreme decays")
