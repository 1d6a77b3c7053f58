"""GPU parity of gdn_scan_varlen against the oracle, through the C ABI.

Every path (DECODE, SEQ) runs in both input modes (fused: norms and gates in-kernel; prepared:
from gdn_prepare_qk_gates) on the five workloads at full size, in the launch configuration the
benchmark uses (plus the benchmark's speculative verification step); the oracle computes sampled
heads and columns of the same launch.  Outputs use
the dtype tolerance (1e-4 fp32, 2e-2 half) and the final fp32 state 1e-4 on the token-sequential
paths; the chunked form uses its own tolerances for both (bf16 2e-2, fp16 1.5e-3)."""
import dataclasses

import numpy as np
import pytest

import cases
import oracle
import workloads
from gpu_util import (CHUNK_SEQ_TOL, CHUNK_SLICE_TOL, CHUNK_TOL, SEQ_STATE_TOL, TOL, assert_close, out_tol, assert_close_slices, state_tol, bits, dev, dev_i32, ensure_built, f64, head_subproblem, require_gpu,
                      sentinel)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def gpu_scan(torch, w, path, prepared, offsets=None, state=None, inplace=False, dev_status=None, use_state=True,
             workspace=None):
    import gated_delta_rule_varlen_amd as gdn

    qkv = dev(w.qkv, w.io)
    a, b = dev(w.a, w.gate_dtype), dev(w.b, w.gate_dtype)
    A_log, dtb = dev(w.A_log, "f32"), dev(w.dt_bias, "f32")
    qk = gb = None
    if prepared:
        qk, gb = gdn.prepare_qk_gates(qkv, HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=a, b=b, A_log=A_log, dt_bias=dtb,
                                      l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid)
    st_in = dev(w.state if state is None else state, "f32") if use_state else None
    out = sentinel((w.N, w.H, w.V), w.io)
    st_out = st_in if (inplace and st_in is not None) else sentinel((w.B, w.H, w.V, w.K), "f32")
    out, st_out, used = gdn.scan_varlen(qkv, dev_i32(w.offsets if offsets is None else offsets), HQ=w.HQ, H=w.H,
                                        K=w.K, V=w.V, a=a, b=b, A_log=A_log, dt_bias=dtb, state_in=st_in,
                                        qk_prep=qk, gb_prep=gb, l2norm=w.l2norm, softplus=w.softplus,
                                        sigmoid=w.sigmoid, scale=w.scale, path=path, out=out, state_out=st_out,
                                        dev_status=dev_status, workspace=workspace)
    torch.cuda.synchronize()
    return out, st_out, used


# (workload, heads sampled (None = all), columns sampled per head (None = all))
SAMPLES = {
    "tiny_fp32": (None, None),
    "decode": ([0, 1, 17, 31], None),
    "prefill": ([0, 13, 31], None),
    "long": ([0, 9], [0, 1, 37, 64, 100, 127]),
    "edge_fp16": (None, None),
    "verify": ([0, 5, 31], None),
    "mixed": ([0, 17, 31], None),
}
PARITY = [(n, p, m) for n in cases.ALL for p in ("decode", "seq") for m in ("fused", "prepared")
          if not (n == "long" and p == "decode")]
# the chunked path runs on fused bf16/fp16 inputs with the softplus gate and L2 norm
PARITY += [("decode", "chunk", "fused"), ("prefill", "chunk", "fused"), ("long", "chunk", "fused")]
# the speculative verification step (B=256 x 5 tokens) at full size: DECODE's short-sequence form and SEQ
PARITY += [("verify", "decode", "fused"), ("verify", "decode", "prepared"), ("verify", "seq", "fused")]
# a serving batch mixing 255 single tokens with one 4096-token prefill, on every path
PARITY += [("mixed", "decode", "fused"), ("mixed", "seq", "fused"), ("mixed", "chunk", "fused"), ("mixed", "auto", "fused")]


def check_against_oracle(w, name, out, st, path):
    heads, cols = SAMPLES[name]
    heads = range(w.H) if heads is None else heads
    og, sg = f64(out), f64(st)
    ref_o, ref_s, got_o, got_s = [], [], [], []
    for h in heads:
        sub, vsel = head_subproblem(w, h, cols)
        o_ref, s_ref = oracle.scan(sub.pop("qkv"), w.offsets, **sub)
        ref_o.append(o_ref[:, 0])
        ref_s.append(s_ref[:, 0])
        got_o.append(og[:, h][:, vsel])
        got_s.append(sg[:, h][:, vsel])
    assert_close(np.stack(got_o), np.stack(ref_o), out_tol(w.io, path), f"{name} {path} out")
    assert_close(np.stack(got_s), np.stack(ref_s), state_tol(w.io, path), f"{name} {path} final state")


@pytest.mark.parametrize("name,path,mode", PARITY)
def test_scan_matches_oracle(torch, name, path, mode):
    w = cases.get(name)
    print(f"[scan parity] {name} path={path} mode={mode} B={w.B} N={w.N} H={w.H} K={w.K} V={w.V}", flush=True)
    out, st, used = gpu_scan(torch, w, path, mode == "prepared")
    assert used == path or path == "auto"
    assert np.all(np.isfinite(f64(out))), "an output element was left unwritten"
    check_against_oracle(w, name, out, st, used)


@pytest.mark.parametrize("name,want", [("tiny_fp32", "seq"), ("decode", "decode"), ("edge_fp16", "seq"),
                                       ("prefill", "chunk"), ("verify", "decode"), ("mixed", "chunk")])
def test_auto_path_choice(torch, name, want):
    w = cases.get(name)
    _, _, used = gpu_scan(torch, w, "auto", False)
    assert used == want


@pytest.mark.parametrize("name,path", [("tiny_fp32", "seq"), ("edge_fp16", "seq"), ("decode", "decode"),
                                       ("prefill", "chunk")])
def test_in_place_state_and_determinism(torch, name, path):
    w = cases.get(name)
    o1, s1, _ = gpu_scan(torch, w, path, False)
    o2, s2, _ = gpu_scan(torch, w, path, False)
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(s1), bits(s2)), "not deterministic"
    o3, s3, _ = gpu_scan(torch, w, path, False, inplace=True)
    assert np.array_equal(bits(o1), bits(o3)) and np.array_equal(bits(s1), bits(s3)), "in-place update differs"


def test_zero_length_sequences_copy_state_bit_exactly(torch):
    w = cases.get("edge_fp16")
    empty = np.flatnonzero(w.lengths == 0)
    assert len(empty) >= 3
    for path in ("seq", "decode"):
        _, st, _ = gpu_scan(torch, w, path, False)
        assert np.array_equal(bits(st)[empty], w.state[empty].view(np.int32))


def test_null_initial_state_is_zero_state(torch):
    w = cases.get("tiny_fp32")
    wz = dataclasses.replace(w, state=np.zeros((w.B, w.H, w.V, w.K), np.float32))
    o1, s1, _ = gpu_scan(torch, wz, "seq", False)
    o2, s2, _ = gpu_scan(torch, wz, "seq", False, use_state=False)
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(s1), bits(s2))


@pytest.mark.parametrize("name,path", [("tiny_fp32", "seq"), ("edge_fp16", "decode"), ("edge_fp16", "seq"),
                                       ("chunk_ragged", "chunk")])
def test_malformed_offsets_write_nothing(torch, name, path):
    w = chunk_ragged(128) if name == "chunk_ragged" else cases.get(name)
    status = torch.full((1,), 777, dtype=torch.int32, device="cuda")
    gpu_scan(torch, w, path, False, dev_status=status)
    assert int(status.item()) == 0
    for case, bad in workloads.malformed_offsets(w.offsets):
        print(f"[scan malformed] {name} {path} {case}", flush=True)
        out, st, _ = gpu_scan(torch, w, path, False, offsets=bad, dev_status=status)
        assert int(status.item()) == -9, case
        assert np.all(bits(out) == bits(sentinel(tuple(out.shape), w.io))), case
        assert np.all(bits(st) == bits(sentinel(tuple(st.shape), "f32"))), case


def test_ragged_multi_tile_small_case(torch):
    # several column tiles per head, a ragged column tail (V not a multiple of the tile), GQA 4,
    # a long and a zero-length sequence: the oracle computes everything
    w = workloads.make(name="ragged", seed=11, lengths=[0, 130, 1, 0, 77], HQ=2, H=8, K=64, V=42, io="bf16",
                       conv_state_dtype="f32")
    for path in ("seq", "decode"):
        for prepared in (False, True):
            out, st, used = gpu_scan(torch, w, path, prepared)
            assert used == path
            o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                                       gate_dtype=w.gate_dtype, a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias,
                                       state_in=w.state)
            assert_close(f64(out), o_ref, TOL[w.io], f"ragged {path} {prepared} out")
            assert_close(f64(st), s_ref, SEQ_STATE_TOL, f"ragged {path} {prepared} state")
            assert_close_slices(f64(out), o_ref, w.lengths, TOL[w.io], f"ragged {path} {prepared} out")


def chunk_ragged(K, H=4, io="bf16", seed=12, G=2):
    """Several chunks per sequence with ragged tails, a one-token and two zero-length sequences,
    G value heads per key head (the chunked form stores q^ and k^ once per key head): every shape
    corner of the chunked path.  With H*V/64 >= 256/7 value-column blocks the state kernel takes its
    64-column tile, else its 16-column tile."""
    return workloads.make(name=f"chunk_ragged_k{K}_h{H}_g{G}_{io}", seed=seed, lengths=[130, 0, 64, 1, 0, 200, 63],
                          HQ=H // G, H=H, K=K, V=K, io=io, conv_state_dtype="f32")


@pytest.mark.parametrize("K,H,io,G", [(64, 4, "bf16", 2), (128, 4, "bf16", 2), (128, 4, "f16", 2), (64, 64, "bf16", 2),
                                      (128, 32, "f16", 2), (128, 4, "bf16", 1), (128, 8, "bf16", 4),
                                      (64, 8, "f16", 8), (128, 64, "bf16", 4)])
def test_chunk_ragged_against_oracle_and_seq(torch, K, H, io, G):
    w = chunk_ragged(K, H, io, G=G)
    print(f"[chunk ragged] K={K} H={H} G={G} {io} N={w.N}", flush=True)
    out_c, st_c, used = gpu_scan(torch, w, "chunk", False)
    assert used == "chunk"
    out_s, st_s, _ = gpu_scan(torch, w, "seq", False)
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                               a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state)
    # fp16: the chunked form on fp16 operands stays within 1e-3 of the oracle
    e1 = assert_close(f64(out_c), o_ref, 1e-3 if w.io == "f16" else CHUNK_TOL[w.io], "chunk out")
    e2 = assert_close(f64(st_c), s_ref, CHUNK_TOL[w.io], "chunk state")
    # the chunked form agrees with the sequential form on the same launch inputs
    e3 = assert_close(f64(out_c), f64(out_s), CHUNK_SEQ_TOL[w.io], "chunk vs seq out")
    e4 = assert_close(f64(st_c), f64(st_s), CHUNK_SEQ_TOL[w.io], "chunk vs seq state")
    print(f"  errors: out {e1:.2e} state {e2:.2e} vs-seq out {e3:.2e} state {e4:.2e}", flush=True)
    empty = np.flatnonzero(w.lengths == 0)
    assert np.array_equal(bits(st_c)[empty], w.state[empty].view(np.int32))


@pytest.mark.parametrize("B", [1023, 1024, 1500])
def test_chunk_many_sequences_against_oracle_and_seq(torch, B):
    # the chunk tables are formed in LDS by one thread per sequence below 1024 sequences and by the
    # looped block scans from 1024 on: both forms, at and around the boundary, with zero-length
    # sequences, one-token sequences and sequences of one and two chunks
    rng = np.random.default_rng(900 + B)
    lengths = rng.integers(0, 100, size=B)
    lengths[rng.choice(B, size=B // 10, replace=False)] = 0
    lengths[rng.choice(B, size=B // 20, replace=False)] = 1
    w = workloads.make(name=f"chunk_many_b{B}", seed=901 + B, lengths=lengths, HQ=1, H=2, K=64, V=64, io="bf16",
                       conv_state_dtype="f32")
    print(f"[chunk many] B={B} N={w.N}", flush=True)
    status = torch.full((1,), 777, dtype=torch.int32, device="cuda")
    out_c, st_c, used = gpu_scan(torch, w, "chunk", False, dev_status=status)
    assert used == "chunk" and int(status.item()) == 0
    out_s, st_s, _ = gpu_scan(torch, w, "seq", False)
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                               a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state)
    e1 = assert_close(f64(out_c), o_ref, CHUNK_TOL[w.io], "chunk out")
    e2 = assert_close(f64(st_c), s_ref, CHUNK_TOL[w.io], "chunk state")
    assert_close_slices(f64(out_c), o_ref, w.lengths, CHUNK_SLICE_TOL[w.io], "chunk out")
    e3 = assert_close(f64(out_c), f64(out_s), CHUNK_SEQ_TOL[w.io], "chunk vs seq out")
    e4 = assert_close(f64(st_c), f64(st_s), CHUNK_SEQ_TOL[w.io], "chunk vs seq state")
    print(f"  errors: out {e1:.2e} state {e2:.2e} vs-seq out {e3:.2e} state {e4:.2e}", flush=True)
    empty = np.flatnonzero(w.lengths == 0)
    assert np.array_equal(bits(st_c)[empty], w.state[empty].view(np.int32))
    # malformed offsets on either form of the tables: nothing is written
    for case, bad in workloads.malformed_offsets(w.offsets):
        print(f"  malformed {case}", flush=True)
        out, st, _ = gpu_scan(torch, w, "chunk", False, offsets=bad, dev_status=status)
        assert int(status.item()) == -9, case
        assert np.all(bits(out) == bits(sentinel(tuple(out.shape), w.io))), case
        assert np.all(bits(st) == bits(sentinel(tuple(st.shape), "f32"))), case


def test_chunk_matches_seq_at_full_prefill_size(torch):
    w = cases.get("prefill")
    out_c, st_c, _ = gpu_scan(torch, w, "chunk", False)
    out_s, st_s, _ = gpu_scan(torch, w, "seq", False)
    e1 = assert_close(f64(out_c), f64(out_s), CHUNK_SEQ_TOL[w.io], "chunk vs seq out")
    e2 = assert_close(f64(st_c), f64(st_s), CHUNK_SEQ_TOL[w.io], "chunk vs seq state")
    print(f"  prefill chunk vs seq: out {e1:.2e} state {e2:.2e}", flush=True)


def test_chunk_rejects_ineligible_inputs(torch):
    import gated_delta_rule_varlen_amd as gdn

    for name in ("tiny_fp32", "edge_fp16"):  # fp32 I/O; no L2 norm / raw log-decay
        w = cases.get(name)
        with pytest.raises(gdn.GdnError) as ei:
            gpu_scan(torch, w, "chunk", False)
        assert ei.value.status == -6
    w = cases.get("prefill")
    with pytest.raises(gdn.GdnError) as ei:  # prepared inputs carry g, not log g
        gpu_scan(torch, w, "chunk", True)
    assert ei.value.status == -6


def test_chunk_segments_with_partial_block_rounds(torch):
    """Three sequences (6000, 900 and 2500 tokens) at H = 12, G = 3, K = V = 128: the first and the
    last are cut into segments (6 and 3 of 16 chunks) and the second is not, and the tmat and combine
    grids end in a partial round of the per-XCD block grouping (12 heads of a chunk; 16 combine
    blocks of a head), whose blocks keep their index.  Against the oracle and the sequential form."""
    w = workloads.make(name="chunk_seg_h12", seed=143, lengths=[6000, 900, 2500], HQ=4, H=12, K=128, V=128, io="bf16",
                       conv_state_dtype="f32", state_std=0.1)
    out_c, st_c, used = gpu_scan(torch, w, "chunk", False)
    assert used == "chunk"
    out_s, st_s, _ = gpu_scan(torch, w, "seq", False)
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                               a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state)
    e1 = assert_close(f64(out_c), o_ref, CHUNK_TOL[w.io], "chunk out")
    e2 = assert_close(f64(st_c), s_ref, CHUNK_TOL[w.io], "chunk state")
    e3 = assert_close(f64(out_c), f64(out_s), CHUNK_SEQ_TOL[w.io], "chunk vs seq out")
    e4 = assert_close(f64(st_c), f64(st_s), CHUNK_SEQ_TOL[w.io], "chunk vs seq state")
    print(f"  segments h12: out {e1:.2e} state {e2:.2e} vs-seq {e3:.2e} / {e4:.2e}", flush=True)


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_chunk_long_sequence_k64(torch, io):
    """One 8192-token sequence (128 chunks in one serial chain) at K = V = 64, both half types:
    the chunked form against the oracle and against the sequential form on the same inputs."""
    w = workloads.make(name=f"chunk_long_k64_{io}", seed=141, lengths=[8192], HQ=4, H=8, K=64, V=64, io=io,
                       conv_state_dtype="f32")
    out_c, st_c, used = gpu_scan(torch, w, "chunk", False)
    assert used == "chunk"
    out_s, st_s, _ = gpu_scan(torch, w, "seq", False)
    o_ref, s_ref = oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                               a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state)
    e1 = assert_close(f64(out_c), o_ref, 1e-3 if w.io == "f16" else CHUNK_TOL[w.io], "chunk out")
    e2 = assert_close(f64(st_c), s_ref, CHUNK_TOL[w.io], "chunk state")
    e3 = assert_close(f64(out_c), f64(out_s), CHUNK_SEQ_TOL[w.io], "chunk vs seq out")
    print(f"  long k64 {io}: out {e1:.2e} state {e2:.2e} vs-seq {e3:.2e}", flush=True)
