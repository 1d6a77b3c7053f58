"""GPU tests of the speculative-decoding capture entry points (gdn_conv1d_varlen_capture,
gdn_scan_varlen_capture) through the C ABI.

* The capture changes nothing else: outputs, final state and new window are bit-identical to the
  calls without capture.
* The recorded conv rows are bit copies of the input rows (exact against the oracle), with zeros
  in the unused slots, for counts below, at and above the capacity and the sequence length, zero
  and negative counts, and empty sequences.
* The recurrence capsule (g, k^, delta) matches the oracle's within the I/O tolerance on the DECODE
  and SEQ paths (the single-token streaming form included), fused and prepared inputs, GQA ratios,
  key widths, ragged column tiles and the rules without the retrieval term; unused slots are exact
  zeros; an inactive step records zeros only.
* The chunked form records from its first chunk (capacities 4, 16 and 64, counts past the
  capacity and the length): capsule against the oracle, outputs and state bit-identical to the
  call without capture; AUTO keeps a prefill-shaped capture on the chunked form, and a capacity
  past one chunk goes to SEQ (forced CHUNK: unsupported).
* Replaying the recorded updates from the initial state reaches the state a run over the accepted
  prefix produces, at the size of a speculative verification step.
* Malformed offsets write nothing."""
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import CHUNK_TOL, TOL, assert_close, bits, dev, dev_i32, ensure_built, f64, require_gpu, sentinel

pytestmark = pytest.mark.gpu

CAP = 4


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def counts_for(lengths, seed):
    """Counts spanning the cases: 0, negative, below/at/above both the capacity and the length."""
    rng = np.random.default_rng(seed)
    pool = np.array([0, -2, 1, 2, CAP - 1, CAP, CAP + 3, 100], np.int32)
    c = pool[rng.integers(0, len(pool), size=len(lengths))]
    c[0] = CAP + 3
    return c.astype(np.int32)


# ---- conv capture -----------------------------------------------------------------------------------

CONV_CASES = {
    "bf16_w4": dict(io="bf16", W=4, D=1),
    "f16_w3_d2_f32win": dict(io="f16", W=3, D=2, conv_state_dtype="f32"),
    "f32_w1": dict(io="f32", W=1, D=1),
    "f32_w5_d3_scalar_channels": dict(io="f32", W=5, D=3, K=30, V=30),  # C % 4 != 0: one channel per thread
    "bf16_w12_d2_wide": dict(io="bf16", W=12, D=2, conv_state_dtype="f32"),  # a width past 8: the per-element form
}


@pytest.mark.parametrize("name", sorted(CONV_CASES))
def test_conv_capture_records_input_rows(torch, name):
    import gated_delta_rule_varlen_amd as gdn

    kw = dict(CONV_CASES[name])
    K, V = kw.pop("K", 32), kw.pop("V", 32)
    lengths = [7, 0, 3, 1, 12, 2, 0, 5]
    w = workloads.make(name=name, seed=500 + sorted(CONV_CASES).index(name), lengths=lengths, HQ=1, H=1, K=K, V=V,
                       **kw)
    counts = counts_for(lengths, 7)
    print(f"[capture conv] {name} C={w.C} counts={counts.tolist()}", flush=True)
    x, cw, cb = dev(w.x, w.io), dev(w.conv_w, w.io), dev(w.conv_bias, w.io)
    cst, off = dev(w.conv_state, w.conv_state_dtype), dev_i32(w.offsets)
    sdt = getattr(torch, {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}[w.conv_state_dtype])
    y1, s1 = gdn.conv1d_varlen(x, cw, off, bias=cb, state_in=cst, dilation=w.D, silu=w.silu, state_dtype=sdt)
    y2, s2, upd = gdn.conv1d_varlen_capture(x, cw, off, cap=CAP, counts=dev_i32(counts), bias=cb, state_in=cst,
                                            dilation=w.D, silu=w.silu, state_dtype=sdt,
                                            updates=sentinel((w.B, CAP, w.C), w.io))
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y2))
    if s1 is not None:
        assert np.array_equal(bits(s1), bits(s2))
    ref = oracle.conv_capture(w.x, w.offsets, counts, cap=CAP, x_dtype=w.io)
    assert np.array_equal(f64(upd), ref)
    assert np.all(bits(upd)[ref == 0] == 0)  # unused slots are +0, not sentinels


def test_conv_capture_malformed_offsets_write_nothing(torch):
    import gated_delta_rule_varlen_amd as gdn

    w = workloads.make(name="cap_conv_bad", seed=510, lengths=[3, 2, 4], HQ=1, H=1, K=32, V=32, io="bf16")
    status = dev_i32(np.array([12345]))
    upd = sentinel((w.B, CAP, w.C), w.io)
    gdn.conv1d_varlen_capture(dev(w.x, w.io), dev(w.conv_w, w.io), dev_i32(np.array([0, 3, 2, 9], np.int32)),
                              cap=CAP, counts=dev_i32(np.array([4, 4, 4])), updates=upd, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.cpu()[0]) == -9
    assert np.all(bits(upd) == bits(sentinel(tuple(upd.shape), w.io)))


# ---- recurrence capture -----------------------------------------------------------------------------

def split(capsule, B, cap, HQ, H, K, V):
    g = capsule[:, :cap * H].reshape(B, cap, H)
    kh = capsule[:, cap * H:cap * (H + HQ * K)].reshape(B, cap, HQ, K)
    d = capsule[:, cap * (H + HQ * K):].reshape(B, cap, H, V)
    return g, kh, d


def run_capture(torch, w, counts, *, path, prepared=False, active=None, retrieve=True, state_out=True):
    import gated_delta_rule_varlen_amd as gdn

    qkv = dev(w.qkv, w.io)
    a, b = dev(w.a, w.gate_dtype), dev(w.b, w.gate_dtype)
    A_log, dtb = dev(w.A_log, "f32"), dev(w.dt_bias, "f32")
    qk = gb = None
    if prepared:
        qk, gb = gdn.prepare_qk_gates(qkv, HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=a, b=b, A_log=A_log, dt_bias=dtb,
                                      l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid)
    common = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=a, b=b, A_log=A_log, dt_bias=dtb, state_in=dev(w.state, "f32"),
                  qk_prep=qk, gb_prep=gb, l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale,
                  path=path, retrieve=retrieve)
    off = dev_i32(w.offsets)
    o1, s1, used1 = gdn.scan_varlen(qkv, off, out=sentinel((w.N, w.H, w.V), w.io),
                                    state_out=sentinel((w.B, w.H, w.V, w.K), "f32") if state_out else None,
                                    write_state=state_out, **common)
    o2, s2, caps, used2 = gdn.scan_varlen_capture(
        qkv, off, cap=CAP, counts=dev_i32(counts), active=None if active is None else dev_i32(np.array([active])),
        capsule=sentinel((w.B, CAP * (w.H + w.HQ * w.K + w.H * w.V)), "f32"), out=sentinel((w.N, w.H, w.V), w.io),
        state_out=sentinel((w.B, w.H, w.V, w.K), "f32") if state_out else None, write_state=state_out, **common)
    torch.cuda.synchronize()
    assert used1 == used2 == path
    assert np.array_equal(bits(o1), bits(o2)), "capture changed the outputs"
    if state_out:
        assert np.array_equal(bits(s1), bits(s2)), "capture changed the final state"
    return f64(caps)


def oracle_capsule(w, counts, active=None, retrieve=True):
    _, _, caps = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                             a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state, l2norm=w.l2norm,
                             softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale, retrieve=retrieve,
                             counts=counts, active=None if active is None else np.array([active], np.int32), cap=CAP)
    return caps


def check_capsule(w, got, ref, tol, what):
    B, HQ, H, K, V = w.B, w.HQ, w.H, w.K, w.V
    assert np.all(got[ref == 0] == 0), f"{what}: unused slots must be zero"
    for part, gp, rp in zip(("g", "k^", "delta"), split(got, B, CAP, HQ, H, K, V), split(ref, B, CAP, HQ, H, K, V)):
        assert_close(gp, rp, tol, f"{what} {part}")


SCAN_CASES = {
    # lengths mix single tokens, speculative blocks of 2..6 tokens and an empty sequence
    "bf16_k128_g2": dict(HQ=2, H=4, K=128, V=128, io="bf16"),
    "f32_k64_g1": dict(HQ=2, H=2, K=64, V=64, io="f32"),
    "f16_k256_g4_v32": dict(HQ=1, H=4, K=256, V=32, io="f16"),
    "f32_k32_v36_ragged_tile": dict(HQ=1, H=2, K=32, V=36, io="f32"),
    "bf16_k64_raw_gates": dict(HQ=2, H=2, K=64, V=64, io="bf16", softplus=False, sigmoid=False, l2norm=False,
                               decay_range=(-1.0, 0.0), beta_range=(0.0, 1.0), unit_k_scan=True),
}
LENS = [5, 1, 0, 3, 6, 1, 2, 4]


@pytest.mark.parametrize("name", sorted(SCAN_CASES))
@pytest.mark.parametrize("path", ["decode", "seq"])
def test_scan_capture_matches_oracle(torch, name, path):
    w = workloads.make(name=name, seed=520 + sorted(SCAN_CASES).index(name), lengths=LENS, **SCAN_CASES[name])
    counts = counts_for(LENS, 11)
    print(f"[capture scan] {name} {path} counts={counts.tolist()}", flush=True)
    got = run_capture(torch, w, counts, path=path)
    check_capsule(w, got, oracle_capsule(w, counts), TOL[w.io], f"{name}/{path}")


@pytest.mark.parametrize("path", ["decode", "seq"])
@pytest.mark.parametrize("retrieve", [True, False])
def test_scan_capture_prepared_inputs_and_rules(torch, path, retrieve):
    w = workloads.make(name="cap_prep", seed=540, lengths=LENS, HQ=2, H=4, K=64, V=64, io="f32")
    counts = counts_for(LENS, 13)
    got = run_capture(torch, w, counts, path=path, prepared=True, retrieve=retrieve)
    check_capsule(w, got, oracle_capsule(w, counts, retrieve=retrieve), TOL[w.io], f"prepared/{path}/{retrieve}")


def test_scan_capture_single_token_streaming_blocks(torch):
    """Decode-step shape (one token per sequence, carried state, whole column tiles): the streaming
    form of the DECODE kernel records slot 0."""
    lens = [1] * 12 + [0, 1]
    w = workloads.make(name="cap_stream", seed=541, lengths=lens, HQ=2, H=4, K=128, V=128, io="bf16")
    counts = np.array([1, 2, 0, 4, -1, 1, 3, 1, 1, 0, 5, 1, 1, 1], np.int32)
    got = run_capture(torch, w, counts, path="decode")
    check_capsule(w, got, oracle_capsule(w, counts), TOL[w.io], "stream")


@pytest.mark.parametrize("path", ["decode", "seq"])
def test_scan_capture_inactive_records_zeros(torch, path):
    w = workloads.make(name="cap_inactive", seed=542, lengths=LENS, HQ=2, H=4, K=64, V=64, io="bf16")
    counts = np.full(len(LENS), CAP, np.int32)
    got = run_capture(torch, w, counts, path=path, active=0)
    assert not got.any()
    got = run_capture(torch, w, counts, path=path, active=1)
    check_capsule(w, got, oracle_capsule(w, counts, active=1), TOL[w.io], "active")


def test_scan_capture_without_final_state(torch):
    w = workloads.make(name="cap_nostate", seed=543, lengths=LENS, HQ=1, H=2, K=128, V=64, io="bf16")
    counts = counts_for(LENS, 17)
    for path in ("decode", "seq"):
        got = run_capture(torch, w, counts, path=path, state_out=False)
        check_capsule(w, got, oracle_capsule(w, counts), TOL[w.io], f"nostate/{path}")


def test_auto_path_records_on_the_chunked_form(torch):
    """A prefill-shaped call that AUTO gives to the chunked form records there (the capacity fits one
    chunk); a capacity past one chunk sends it to the token-sequential form."""
    import gated_delta_rule_varlen_amd as gdn

    w = workloads.make(name="cap_auto", seed=544, lengths=[200, 150], HQ=1, H=2, K=64, V=64, io="bf16")
    qkv = dev(w.qkv, w.io)
    kw = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype),
              A_log=dev(w.A_log, "f32"), dt_bias=dev(w.dt_bias, "f32"), state_in=dev(w.state, "f32"))
    for cap, counts, path in ((CAP, np.array([CAP, 2], np.int32), "chunk"), (65, np.array([65, 70], np.int32), "seq")):
        _, _, caps, used = gdn.scan_varlen_capture(qkv, dev_i32(w.offsets), cap=cap, counts=dev_i32(counts), **kw)
        torch.cuda.synchronize()
        assert used == path
        _, _, ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                                gate_dtype=w.gate_dtype, a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias,
                                state_in=w.state, counts=counts, cap=cap)
        got = f64(caps)
        assert np.all(got[ref == 0] == 0)
        assert_close(got, ref, CHUNK_TOL[w.io] if path == "chunk" else TOL[w.io], f"auto cap={cap}")


CHUNK_CAPTURE_CASES = {
    # (lengths, counts, cap, geometry): first chunks cut short, whole, and past the capacity
    "bf16_k128_g2_cap64": ([70, 5, 0, 130, 1, 64, 3], [64, 5, 4, 80, 1, 63, -1], 64,
                           dict(HQ=2, H=4, K=128, V=128, io="bf16")),
    "f16_k64_g1_cap16": ([20, 0, 200, 7, 16], [16, 3, 9, 100, 16], 16, dict(HQ=2, H=2, K=64, V=64, io="f16")),
    "bf16_k64_g4_cap4": ([100, 2, 64, 65], [4, 4, 0, 3], 4, dict(HQ=1, H=4, K=64, V=64, io="bf16")),
}


@pytest.mark.parametrize("name", sorted(CHUNK_CAPTURE_CASES))
def test_chunk_capture_matches_oracle(torch, name):
    """The chunked form records g, k^ and delta (rows of its U = T R, the per-token deltas) of the
    first chunk; the capsule matches the oracle to the half-precision tolerance and recording
    changes neither outputs nor final state (bit for bit)."""
    import gated_delta_rule_varlen_amd as gdn

    lens, counts, cap, geo = CHUNK_CAPTURE_CASES[name]
    w = workloads.make(name=name, seed=570 + sorted(CHUNK_CAPTURE_CASES).index(name), lengths=lens, **geo)
    counts = np.array(counts, np.int32)
    print(f"[capture chunk] {name} cap={cap} counts={counts.tolist()}", flush=True)
    qkv = dev(w.qkv, w.io)
    kw = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype),
              A_log=dev(w.A_log, "f32"), dt_bias=dev(w.dt_bias, "f32"), state_in=dev(w.state, "f32"), path="chunk")
    off = dev_i32(w.offsets)
    o1, s1, used1 = gdn.scan_varlen(qkv, off, out=sentinel((w.N, w.H, w.V), w.io),
                                    state_out=sentinel((w.B, w.H, w.V, w.K), "f32"), **kw)
    o2, s2, caps, used2 = gdn.scan_varlen_capture(
        qkv, off, cap=cap, counts=dev_i32(counts),
        capsule=sentinel((w.B, cap * (w.H + w.HQ * w.K + w.H * w.V)), "f32"), out=sentinel((w.N, w.H, w.V), w.io),
        state_out=sentinel((w.B, w.H, w.V, w.K), "f32"), **kw)
    torch.cuda.synchronize()
    assert used1 == used2 == "chunk"
    assert np.array_equal(bits(o1), bits(o2)), "capture changed the outputs"
    assert np.array_equal(bits(s1), bits(s2)), "capture changed the final state"
    _, _, ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                            a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state, counts=counts, cap=cap)
    got = f64(caps)
    assert np.all(got[ref == 0] == 0), "unused slots must be zero"
    g_n, k_n = cap * w.H, cap * (w.H + w.HQ * w.K)
    for part, sl in (("g", slice(0, g_n)), ("k^", slice(g_n, k_n)), ("delta", slice(k_n, None))):
        assert_close(got[:, sl], ref[:, sl], CHUNK_TOL[w.io], f"{name} {part}")


def test_chunk_capture_past_one_chunk_is_unsupported(torch):
    import gated_delta_rule_varlen_amd as gdn
    from gated_delta_rule_varlen_amd import _abi

    w = workloads.make(name="cap_chunk65", seed=575, lengths=[100, 70], HQ=1, H=2, K=64, V=64, io="bf16")
    with pytest.raises(gdn.GdnError) as e:
        gdn.scan_varlen_capture(dev(w.qkv, w.io), dev_i32(w.offsets), cap=65, counts=dev_i32(np.array([65, 65], np.int32)),
                                HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype),
                                A_log=dev(w.A_log, "f32"), dt_bias=dev(w.dt_bias, "f32"), path="chunk")
    assert e.value.status == _abi.ERR_UNSUPPORTED


def test_scan_capture_malformed_offsets_write_nothing(torch):
    import gated_delta_rule_varlen_amd as gdn

    w = workloads.make(name="cap_bad", seed=545, lengths=[3, 2, 4], HQ=1, H=2, K=64, V=64, io="bf16")
    for path in ("decode", "seq"):
        status = dev_i32(np.array([12345]))
        caps = sentinel((w.B, CAP * (w.H + w.HQ * w.K + w.H * w.V)), "f32")
        gdn.scan_varlen_capture(dev(w.qkv, w.io), dev_i32(np.array([0, 3, 2, 9], np.int32)), cap=CAP,
                                counts=dev_i32(np.array([4, 4, 4])), capsule=caps, HQ=w.HQ, H=w.H, K=w.K, V=w.V,
                                a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"),
                                dt_bias=dev(w.dt_bias, "f32"), path=path, dev_status=status)
        torch.cuda.synchronize()
        assert int(status.cpu()[0]) == -9
        assert np.all(bits(caps) == bits(sentinel(tuple(caps.shape), "f32")))


def test_speculative_verification_step_replay(torch):
    """A verification step at model size (B=64 sequences of 5 tokens: the last accepted token and 4
    drafts; HQ=16, H=32, K=V=128, bf16): conv and recurrence record up to 4 tokens; replaying the
    recorded updates of the accepted prefix from the initial state on the device reaches the final
    state of a second run over the accepted prefix only, and the recorded conv rows equal the
    inputs.  Sampled sequences are checked against the oracle."""
    import gated_delta_rule_varlen_amd as gdn

    B, T, HQ, H, K, V = 64, 5, 16, 32, 128, 128
    w = workloads.make(name="cap_verify", seed=546, lengths=[T] * B, HQ=HQ, H=H, K=K, V=V, io="bf16",
                       conv_state_dtype="f32")
    rng = np.random.default_rng(547)
    accepted = rng.integers(0, CAP + 1, size=B).astype(np.int32)  # tokens the verifier keeps
    x, off = dev(w.x, w.io), dev_i32(w.offsets)
    cnt = dev_i32(accepted)
    y, _, upd = gdn.conv1d_varlen_capture(x, dev(w.conv_w, w.io), off, cap=CAP, counts=cnt,
                                          bias=dev(w.conv_bias, w.io), state_in=dev(w.conv_state, "f32"),
                                          silu=w.silu, state_dtype=torch.float32)
    A = dict(a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"),
             dt_bias=dev(w.dt_bias, "f32"))
    S0 = dev(w.state, "f32")
    _, _, caps, used = gdn.scan_varlen_capture(y, off, cap=CAP, counts=cnt, HQ=HQ, H=H, K=K, V=V, state_in=S0, **A)
    assert used == "decode"  # at most 8 tokens per sequence on average
    # replay on the device in fp32 (torch: plumbing for the check only)
    g = caps[:, :CAP * H].reshape(B, CAP, H)
    kh = caps[:, CAP * H:CAP * (H + HQ * K)].reshape(B, CAP, HQ, K).repeat_interleave(H // HQ, dim=2)
    d = caps[:, CAP * (H + HQ * K):].reshape(B, CAP, H, V)
    S = S0.clone()
    for i in range(CAP):
        live = (torch.from_numpy(accepted).cuda() > i).float()[:, None, None, None]
        step = g[:, i, :, None, None] * S + d[:, i, :, :, None] * kh[:, i, :, None, :]
        S = live * step + (1 - live) * S
    # second run over the accepted prefix of every sequence (same conv outputs)
    lens = accepted.astype(np.int64)
    toff = workloads.offsets_from_lengths(lens)
    rows = np.concatenate([np.arange(w.offsets[i], w.offsets[i] + lens[i]) for i in range(B)]).astype(np.int64)
    ridx = torch.from_numpy(rows).cuda()
    _, S_ref, _ = gdn.scan_varlen(y.index_select(0, ridx).contiguous(), dev_i32(toff), HQ=HQ, H=H, K=K, V=V,
                                  state_in=S0, path="seq", a=A["a"].index_select(0, ridx).contiguous(),
                                  b=A["b"].index_select(0, ridx).contiguous(), A_log=A["A_log"], dt_bias=A["dt_bias"])
    torch.cuda.synchronize()
    err = assert_close(f64(S), f64(S_ref), 1e-4, "replayed state")
    # conv record: the input rows
    ref_upd = oracle.conv_capture(w.x, w.offsets, accepted, cap=CAP, x_dtype=w.io)
    assert np.array_equal(f64(upd), ref_upd)
    # oracle capsule on 4 sampled sequences (the device conv output as the recurrence's input)
    y_raw = bits(y).view(np.uint16)
    for bsel in (0, 17, 40, 63):
        sl = slice(w.offsets[bsel], w.offsets[bsel + 1])
        _, _, cref = oracle.scan(np.ascontiguousarray(y_raw[sl]), np.array([0, T], np.int32), HQ=HQ, H=H, K=K, V=V,
                                 qkv_dtype="bf16", gate_dtype=w.gate_dtype, a=w.a[sl], b=w.b[sl], A_log=w.A_log,
                                 dt_bias=w.dt_bias, state_in=w.state[bsel:bsel + 1], l2norm=True, softplus=True,
                                 sigmoid=True, counts=accepted[bsel:bsel + 1], cap=CAP)
        check_capsule(SimpleNamespace(B=1, HQ=HQ, H=H, K=K, V=V), f64(caps)[bsel:bsel + 1], cref, TOL["bf16"], f"verify b={bsel}")
    print(f"  replay err {err:.2e}", flush=True)


@pytest.mark.parametrize("path", ["decode", "seq"])
def test_capture_at_capacity_eight(torch, path):
    """cap = 8 (the capacity the pages' speculative decoding uses at most): sequences shorter than,
    equal to and longer than the capacity, recorded in full, on both token-sequential paths (the
    DECODE path's short form carries the sequences of up to 8 tokens)."""
    import gated_delta_rule_varlen_amd as gdn

    cap = 8
    lens = [8, 3, 12, 8, 0, 9, 5, 1]
    w = workloads.make(name=f"cap8_{path}", seed=560, lengths=lens, HQ=2, H=4, K=128, V=128, io="bf16")
    counts = np.array([8, 8, 8, 5, 8, 100, 0, 8], np.int32)
    qkv = dev(w.qkv, w.io)
    kw = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype),
              A_log=dev(w.A_log, "f32"), dt_bias=dev(w.dt_bias, "f32"), state_in=dev(w.state, "f32"), path=path)
    _, _, caps, used = gdn.scan_varlen_capture(qkv, dev_i32(w.offsets), cap=cap, counts=dev_i32(counts), **kw)
    torch.cuda.synchronize()
    assert used == path
    _, _, ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                            a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state, counts=counts, cap=cap)
    got = f64(caps)
    assert np.all(got[ref == 0] == 0)
    g_n, k_n = cap * w.H, cap * (w.H + w.HQ * w.K)
    for part, sl in (("g", slice(0, g_n)), ("k^", slice(g_n, k_n)), ("delta", slice(k_n, None))):
        assert_close(got[:, sl], ref[:, sl], TOL[w.io], f"cap8 {path} {part}")
    upd = gdn.conv1d_varlen_capture(dev(w.x, w.io), dev(w.conv_w, w.io), dev_i32(w.offsets), cap=cap,
                                    counts=dev_i32(counts), bias=dev(w.conv_bias, w.io),
                                    state_in=dev(w.conv_state, w.conv_state_dtype), silu=w.silu,
                                    state_dtype=getattr(torch, {"f32": "float32", "bf16": "bfloat16"}[w.conv_state_dtype]))[2]
    torch.cuda.synchronize()
    assert np.array_equal(f64(upd), oracle.conv_capture(w.x, w.offsets, counts, cap=cap, x_dtype=w.io))
