"""GPU parity on seeded random shapes and flags, against the oracle.

* Recurrence, every path: each case draws a batch size, ragged lengths (empty and one-token
  sequences included), key heads, value heads per key head (1, 2 or 4), K = V in {64, 128} and a
  half-precision dtype, then runs DECODE, SEQ and CHUNK on the same inputs.
* Recurrence, wider flags (DECODE and SEQ): fp32 I/O, K != V, raw decay and rate inputs, no q/k
  normalisation, prepared inputs.
* CHUNK gate inputs: raw rates, no rate input, fp32 gate inputs (against the oracle and SEQ).
* Conv: widths 1..8, dilations 1..3, channel counts off the 16-byte vector width, every dtype with
  its own or an fp32 window, bias and SiLU on or off, sequences shorter than the window.
* Single-launch decode step: bit-identical to the two calls, on batches either side of its
  small-grid launch.
* Speculative-decoding capture on random batches, lengths and counts.
* Every entry point on a batch of empty sequences (N = 0).
Outputs and final state are held to the dtype tolerance; the state of an empty sequence and the
carried conv window must come back bit-identical."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import CHUNK_SEQ_TOL, CHUNK_SLICE_TOL, CHUNK_TOL, SEQ_STATE_TOL, TOL, out_tol, assert_close, assert_close_slices, state_tol, bits, dev, dev_i32, ensure_built, f64, require_gpu
from test_gpu_scan import gpu_scan

pytestmark = pytest.mark.gpu

SEEDS = list(range(301, 317))


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def draw(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    lengths = rng.integers(0, 261, size=B)
    kind = rng.random(B)
    lengths[kind < 0.2] = 0
    lengths[(kind >= 0.2) & (kind < 0.3)] = 1
    G = int(rng.choice([1, 2, 4]))
    HQ = int(rng.choice([1, 2]))
    K = int(rng.choice([64, 128]))
    io = str(rng.choice(["bf16", "f16"]))
    return workloads.make(name=f"random_{seed}", seed=seed, lengths=[int(x) for x in lengths], HQ=HQ, H=HQ * G,
                          K=K, V=K, io=io, conv_state_dtype="f32")


@pytest.fixture(scope="module")
def references():
    refs = {}
    for seed in SEEDS:
        w = draw(seed)
        refs[seed] = (w, oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                                     gate_dtype=w.gate_dtype, a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias,
                                     state_in=w.state))
    return refs


@pytest.mark.parametrize("path", ["decode", "seq", "chunk"])
@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_against_oracle(torch, references, seed, path):
    w, (o_ref, s_ref) = references[seed]
    lens = [int(x) for x in w.lengths]
    print(f"[random {seed}] path={path} B={w.B} lengths={lens} HQ={w.HQ} H={w.H} K={w.K} {w.io}", flush=True)
    out, st, used = gpu_scan(torch, w, path, False)
    assert used == path
    if w.N > 0:
        assert_close(f64(out), o_ref, out_tol(w.io, path), f"{path} out")
        assert_close_slices(f64(out), o_ref, w.lengths, CHUNK_SLICE_TOL[w.io] if path == "chunk" else TOL[w.io],
                            f"{path} out")
    assert_close(f64(st), s_ref, state_tol(w.io, path), f"{path} state")
    assert_close_slices(f64(st), s_ref, w.lengths, CHUNK_SLICE_TOL[w.io] if path == "chunk" else SEQ_STATE_TOL,
                        f"{path} state", token_major=False)
    empty = np.flatnonzero(w.lengths == 0)
    assert np.array_equal(bits(st)[empty], w.state[empty].view(np.int32))


FLAG_SEEDS = list(range(401, 417))


def draw_flags(seed):
    """Wider flag space of the token-sequential paths: fp32 I/O, K != V, raw decay and rate inputs,
    no q/k normalisation (unit-norm keys then keep the recurrence bounded), prepared inputs."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    lengths = rng.integers(0, 140, size=B)
    lengths[rng.random(B) < 0.2] = 0
    G = int(rng.choice([1, 2, 4]))
    HQ = int(rng.choice([1, 2]))
    K = int(rng.choice([32, 64, 128, 256]))
    V = int(rng.choice([32, 64, 128]))
    io = str(rng.choice(["f32", "bf16", "f16"]))
    l2norm = bool(rng.random() < 0.5)
    softplus = bool(rng.random() < 0.5)
    sigmoid = bool(rng.random() < 0.5)
    prepared = bool(rng.random() < 0.5)
    w = workloads.make(name=f"random_flags_{seed}", seed=seed, lengths=[int(x) for x in lengths], HQ=HQ, H=HQ * G,
                       K=K, V=V, io=io, conv_state_dtype="f32", l2norm=l2norm, softplus=softplus, sigmoid=sigmoid,
                       decay_range=None if softplus else (-1.0, 0.0), beta_range=None if sigmoid else (0.0, 1.0),
                       unit_k_scan=not l2norm)
    return w, prepared


@pytest.fixture(scope="module")
def flag_references():
    refs = {}
    for seed in FLAG_SEEDS:
        w, prepared = draw_flags(seed)
        refs[seed] = (w, prepared, oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                                               gate_dtype=w.gate_dtype, a=w.a, b=w.b, A_log=w.A_log,
                                               dt_bias=w.dt_bias, state_in=w.state, l2norm=w.l2norm,
                                               softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale))
    return refs


@pytest.mark.parametrize("path", ["decode", "seq"])
@pytest.mark.parametrize("seed", FLAG_SEEDS)
def test_random_flags_against_oracle(torch, flag_references, seed, path):
    w, prepared, (o_ref, s_ref) = flag_references[seed]
    lens = [int(x) for x in w.lengths]
    print(f"[random flags {seed}] path={path} prepared={prepared} B={w.B} lengths={lens} HQ={w.HQ} H={w.H} "
          f"K={w.K} V={w.V} {w.io} l2norm={w.l2norm} softplus={w.softplus} sigmoid={w.sigmoid}", flush=True)
    out, st, used = gpu_scan(torch, w, path, prepared)
    assert used == path
    if w.N > 0:
        assert_close(f64(out), o_ref, TOL[w.io], f"{path} out")
    assert_close(f64(st), s_ref, SEQ_STATE_TOL, f"{path} state")
    empty = np.flatnonzero(w.lengths == 0)
    assert np.array_equal(bits(st)[empty], w.state[empty].view(np.int32))


CHUNK_GATE_CASES = {
    # the chunked form's gate inputs beyond the sigmoid-of-logits default: raw rates in [0, 1], no
    # rate input (beta = 1), fp32 gate inputs with half-precision q/k/v, and their mixtures
    "raw_rate_bf16_k128_g2": dict(HQ=2, H=4, K=128, V=128, io="bf16", sigmoid=False, beta_range=(0.0, 1.0)),
    "no_rate_f16_k64": dict(HQ=2, H=2, K=64, V=64, io="f16", has_beta=False),
    "f32_gates_bf16_k128": dict(HQ=1, H=2, K=128, V=128, io="bf16", gate_dtype="f32"),
    "f32_raw_rate_f16_k64_g4_no_state": dict(HQ=1, H=4, K=64, V=64, io="f16", gate_dtype="f32", sigmoid=False,
                                             beta_range=(0.0, 1.0), state_std=None),
    "f32_gates_no_rate_bf16_k64": dict(HQ=2, H=4, K=64, V=64, io="bf16", gate_dtype="f32", has_beta=False),
}
CHUNK_GATE_LENS = [200, 64, 1, 0, 130, 65, 17]


@pytest.mark.parametrize("name", sorted(CHUNK_GATE_CASES))
def test_chunk_gate_variants_against_oracle_and_seq(torch, name):
    """CHUNK with raw rates (no sigmoid), without a rate input, and with fp32 gate inputs: outputs
    and final state against the oracle and against SEQ on the same inputs."""
    w = workloads.make(name=name, seed=450 + sorted(CHUNK_GATE_CASES).index(name), lengths=CHUNK_GATE_LENS,
                       **CHUNK_GATE_CASES[name])
    print(f"[chunk gates] {name} lengths={CHUNK_GATE_LENS} b={'none' if w.b is None else w.gate_dtype} "
          f"sigmoid={w.sigmoid}", flush=True)
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                               gate_dtype=w.gate_dtype, a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias,
                               state_in=w.state, l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid,
                               scale=w.scale)
    out, st, used = gpu_scan(torch, w, "chunk", False, use_state=w.state is not None)
    assert used == "chunk"
    assert_close(f64(out), o_ref, CHUNK_TOL[w.io], f"{name} chunk out")
    assert_close_slices(f64(out), o_ref, w.lengths, CHUNK_SLICE_TOL[w.io], f"{name} chunk out")
    assert_close(f64(st), s_ref, CHUNK_TOL[w.io], f"{name} chunk state")
    assert_close_slices(f64(st), s_ref, w.lengths, CHUNK_SLICE_TOL[w.io], f"{name} chunk state", token_major=False)
    o_seq, s_seq, used = gpu_scan(torch, w, "seq", False, use_state=w.state is not None)
    assert used == "seq"
    assert_close(f64(out), f64(o_seq), CHUNK_SEQ_TOL[w.io], f"{name} chunk vs seq out")
    assert_close(f64(st), f64(s_seq), CHUNK_SEQ_TOL[w.io], f"{name} chunk vs seq state")


@pytest.mark.parametrize("path", ["decode", "seq", "chunk"])
def test_negative_scale_is_applied(torch, path):
    """A nonzero scale is applied as given, negative included (only zero selects 1/sqrt(K))."""
    w = workloads.make(name="neg_scale", seed=470, lengths=[90, 3, 0, 70], HQ=2, H=4, K=64, V=64, io="bf16")
    w.scale = -0.4
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                               gate_dtype=w.gate_dtype, a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias,
                               state_in=w.state, scale=w.scale)
    out, st, used = gpu_scan(torch, w, path, False)
    assert used == path
    assert_close(f64(out), o_ref, TOL[w.io], f"{path} out")
    assert_close(f64(st), s_ref, state_tol(w.io, path), f"{path} state")
    assert np.sum(f64(out) * o_ref) > 0  # the sign follows the scale


CONV_SEEDS = list(range(501, 517))


def draw_conv(seed):
    """Random conv calls: widths 1..8, dilations 1..3, channel counts that do and do not fill 16-byte
    vectors, every I/O dtype with its own or an fp32 window, bias and SiLU on or off, short ragged
    sequences (shorter than the window too) and empty ones."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    lengths = rng.integers(0, 41, size=B)
    lengths[rng.random(B) < 0.2] = 0
    HQ = int(rng.choice([1, 2]))
    H = HQ * int(rng.choice([1, 2]))
    K = int(rng.choice([3, 8, 16, 32]))
    V = int(rng.choice([2, 8, 16]))
    io = str(rng.choice(["f32", "bf16", "f16"]))
    return workloads.make(name=f"random_conv_{seed}", seed=seed, lengths=[int(x) for x in lengths], HQ=HQ, H=H,
                          K=K, V=V, W=int(rng.integers(1, 9)), D=int(rng.integers(1, 4)), io=io,
                          conv_state_dtype=str(rng.choice([io, "f32"])), silu=bool(rng.random() < 0.5),
                          has_bias=bool(rng.random() < 0.5))


@pytest.mark.parametrize("seed", CONV_SEEDS)
def test_random_conv_against_oracle(torch, seed):
    from test_gpu_conv import gpu_conv

    w = draw_conv(seed)
    lens = [int(x) for x in w.lengths]
    print(f"[random conv {seed}] B={w.B} lengths={lens} C={w.C} W={w.W} D={w.D} {w.io} window={w.conv_state_dtype} "
          f"bias={w.conv_bias is not None} silu={w.silu}", flush=True)
    y, st = gpu_conv(torch, w)
    y_ref, st_ref = oracle.conv(w.x, w.conv_w, w.offsets, W=w.W, D=w.D, x_dtype=w.io, bias=w.conv_bias,
                                state_in=w.conv_state, silu=w.silu, state_dtype=w.conv_state_dtype)
    if w.N > 0:
        assert_close(f64(y), y_ref, TOL[w.io], "conv y")
    if w.L > 0:
        assert np.array_equal(f64(st), st_ref), "carried window"


STEP_SEEDS = list(range(601, 613))


def draw_step(seed):
    """Random single-launch decode steps: batches on both sides of the small-grid launch (fewer
    blocks than compute units), empty sequences, every key width and dtype, GQA 1..4, conv widths
    1..5 and dilations with a window of at most 4."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 301))
    lengths = (rng.random(B) >= 0.2).astype(int)
    HQ = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4]))
    K = int(rng.choice([32, 64, 128, 256]))
    V = int(rng.choice([4, 32, 64, 128]))
    W = int(rng.integers(1, 6))
    D = int(rng.choice([1, 2])) if W <= 3 else 1
    io = str(rng.choice(["f32", "bf16", "f16"]))
    return workloads.make(name=f"random_step_{seed}", seed=seed, lengths=[int(x) for x in lengths], HQ=HQ,
                          H=HQ * G, K=K, V=V, W=W, D=D, io=io, conv_state_dtype=str(rng.choice([io, "f32"])))


@pytest.mark.parametrize("seed", STEP_SEEDS)
def test_random_decode_step_matches_two_calls(torch, seed):
    from test_gpu_decode_step import run_chain, run_fused

    w = draw_step(seed)
    print(f"[random step {seed}] B={w.B} N={w.N} HQ={w.HQ} H={w.H} K={w.K} V={w.V} W={w.W} D={w.D} {w.io} "
          f"window={w.conv_state_dtype} blocks={w.B * w.HQ}", flush=True)
    o2, s2, c2 = run_chain(torch, w)
    o1, s1, c1 = run_fused(torch, w)
    assert np.array_equal(bits(o1), bits(o2)), "out"
    assert np.array_equal(bits(s1), bits(s2)), "state"
    if w.L > 0:
        assert np.array_equal(bits(c1), bits(c2)), "conv window"


def test_every_entry_point_accepts_a_call_without_tokens(torch):
    """A batch of empty sequences (N = 0): every entry point returns, the final states are the
    initial ones bit for bit, the conv windows are copied, and capture records only zeros."""
    import gated_delta_rule_varlen_amd as gdn

    w = workloads.make(name="all_empty", seed=701, lengths=[0, 0, 0], HQ=2, H=4, K=128, V=128, io="bf16",
                       conv_state_dtype="f32")
    assert w.N == 0
    x, cw, cb = dev(w.x, w.io), dev(w.conv_w, w.io), dev(w.conv_bias, w.io)
    cst, st, off = dev(w.conv_state, "f32"), dev(w.state, "f32"), dev_i32(w.offsets)
    gates = dict(a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"),
                 dt_bias=dev(w.dt_bias, "f32"))
    dims = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V)
    counts = torch.full((w.B,), 2, dtype=torch.int32, device="cuda")
    st_bits, cst_bits = w.state.view(np.int32), w.conv_state.view(np.int32)

    out, s1, c1 = gdn.decode_step(x, cw, off, bias=cb, conv_state_in=cst, state_in=st, **gates, **dims)
    y, c2, upd = gdn.conv1d_varlen_capture(x, cw, off, cap=2, counts=counts, bias=cb, state_in=cst, silu=True,
                                           state_dtype=torch.float32)
    o3, s3, cap3, used3 = gdn.scan_varlen_capture(dev(w.qkv, w.io), off, cap=2, counts=counts, state_in=st,
                                                  **gates, **dims)
    HQK = w.HQ * w.K
    qkv = dev(w.qkv, w.io)
    q, k, v = qkv[:, :HQK], qkv[:, HQK:2 * HQK], qkv[:, 2 * HQK:]
    qk, gb = gdn.prepare_qk_gates_strided(q, k, **gates, **dims)
    results = [(s1, c1)]
    for path in ("decode", "seq", "chunk"):
        o4, s4, used4 = gdn.scan_varlen_strided(q, k, v, off, state_in=st, path=path, **gates, **dims)
        assert used4 == path
        results.append((s4, None))
    torch.cuda.synchronize()
    assert out.numel() == 0 and y.numel() == 0 and o3.numel() == 0 and qk.numel() == 0 and gb.numel() == 0
    for s, c in results + [(s3, c2)]:
        assert np.array_equal(bits(s), st_bits)
        if c is not None:
            assert np.array_equal(bits(c), cst_bits)
    assert not np.any(f64(upd)) and not np.any(f64(cap3))


CAPTURE_SEEDS = list(range(801, 811))


@pytest.mark.parametrize("path", ["decode", "seq"])
@pytest.mark.parametrize("seed", CAPTURE_SEEDS)
def test_random_capture_against_oracle(torch, seed, path):
    """Speculative-decoding capture on random batches: lengths 0..12 (either side of the short
    form's 8 tokens), random per-sequence counts (zero, negative, below and past the capacity and
    the length), any key width and dtype; outputs and state unchanged by the capture."""
    from test_gpu_capture import CAP, check_capsule, oracle_capsule, run_capture

    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lengths = [int(x) for x in rng.integers(0, 13, size=B)]
    counts = rng.integers(-1, CAP + 3, size=B).astype(np.int32)
    HQ = int(rng.choice([1, 2]))
    K = int(rng.choice([32, 64, 128, 256]))
    V = int(rng.choice([32, 64, 128]))
    io = str(rng.choice(["f32", "bf16", "f16"]))
    w = workloads.make(name=f"random_capture_{seed}", seed=seed, lengths=lengths, HQ=HQ,
                       H=HQ * int(rng.choice([1, 2, 4])), K=K, V=V, io=io)
    print(f"[random capture {seed}] {path} B={B} N={w.N} HQ={w.HQ} H={w.H} K={K} V={V} {io}", flush=True)
    got = run_capture(torch, w, counts, path=path)
    check_capsule(w, got, oracle_capsule(w, counts), TOL[w.io], f"random capture {seed}/{path}")
