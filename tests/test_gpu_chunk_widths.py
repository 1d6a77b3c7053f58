"""CHUNK at every key and value width the chunked rule admits, through the C ABI.

The paged_ssm.rs page's host fn delta() runs the chunked kernel for any key and value widths that
are multiples of 8 (keys at most 256), K != V included.  The library compiles key widths 64, 128 and
256 and value parts of 32, 64 and 128 columns; other widths run on the next compiled one with the
keys and columns past them zero, and value widths past 128 run in parts of 128 columns, one block
per part.  These tests hold each combination to the oracle and to SEQ on the same inputs (outputs
and final state, per sequence and head as well), with ragged sequences (empty, single-token,
one-chunk, multi-chunk) and GQA; long sequences at the widths that allow segments run cut into
segments, and a first chunk recorded on CHUNK matches the oracle's capsule."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (CHUNK_SEQ_TOL, CHUNK_SLICE_TOL, CHUNK_TOL, TOL, assert_close, assert_close_slices, bits, dev, dev_i32, ensure_built, f64,
                      require_gpu, sentinel)
from test_gpu_scan import gpu_scan

pytestmark = pytest.mark.gpu

WIDTHS = {
    # the edge configuration's geometry (K = 256, V = 64, GQA 4) with the chunked form's gates
    "k256_v64_f16_g4": dict(HQ=2, H=8, K=256, V=64, io="f16"),
    "k256_v256_bf16": dict(HQ=1, H=2, K=256, V=256, io="bf16"),
    "k128_v64_bf16_g2": dict(HQ=2, H=4, K=128, V=64, io="bf16"),
    "k64_v128_f16": dict(HQ=2, H=2, K=64, V=128, io="f16"),
    "k64_v32_bf16_g2": dict(HQ=1, H=2, K=64, V=32, io="bf16"),
    "k128_v256_f16": dict(HQ=1, H=2, K=128, V=256, io="f16"),
    # padded widths: keys past K and columns past V are zero in the kernels
    "k48_v80_bf16_g2": dict(HQ=2, H=4, K=48, V=80, io="bf16"),
    "k200_v24_f16": dict(HQ=1, H=2, K=200, V=24, io="f16"),
    "k96_v320_bf16": dict(HQ=1, H=2, K=96, V=320, io="bf16"),
    "k8_v8_f16": dict(HQ=1, H=2, K=8, V=8, io="f16"),
}
LENS = [200, 64, 1, 0, 130, 65, 17]


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def reference(w):
    return oracle.scan(w.qkv, w.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                       a=w.a, b=w.b, A_log=w.A_log, dt_bias=w.dt_bias, state_in=w.state)


def check_chunk(torch, w, label):
    o_ref, s_ref = reference(w)
    out, st, used = gpu_scan(torch, w, "chunk", False)
    assert used == "chunk"
    assert_close(f64(out), o_ref, CHUNK_TOL[w.io], f"{label} chunk out")
    assert_close_slices(f64(out), o_ref, w.lengths, CHUNK_SLICE_TOL[w.io], f"{label} chunk out")
    assert_close(f64(st), s_ref, CHUNK_TOL[w.io], f"{label} chunk state")
    assert_close_slices(f64(st), s_ref, w.lengths, CHUNK_SLICE_TOL[w.io], f"{label} chunk state", token_major=False)
    empty = np.flatnonzero(w.lengths == 0)
    assert np.array_equal(bits(st)[empty], w.state[empty].view(np.int32)), "empty sequences keep their state"
    o_seq, s_seq, used = gpu_scan(torch, w, "seq", False)
    assert used == "seq"
    assert_close(f64(out), f64(o_seq), CHUNK_SEQ_TOL[w.io], f"{label} chunk vs seq out")
    assert_close(f64(st), f64(s_seq), CHUNK_SEQ_TOL[w.io], f"{label} chunk vs seq state")


@pytest.mark.parametrize("name", sorted(WIDTHS))
def test_chunk_width_against_oracle_and_seq(torch, name):
    w = workloads.make(name=name, seed=1200 + sorted(WIDTHS).index(name), lengths=LENS, **WIDTHS[name])
    print(f"[chunk width] {name} K={w.K} V={w.V} {w.io} HQ={w.HQ} H={w.H} lengths={LENS}", flush=True)
    check_chunk(torch, w, name)


LONG = {
    # (geometry, lengths): segments at K=128/V=64 and K=64/V=32; one segment per sequence at K=256
    "k128_v64_bf16_segments": (dict(HQ=1, H=2, K=128, V=64, io="bf16"), [3000, 40]),
    "k64_v32_f16_segments": (dict(HQ=2, H=2, K=64, V=32, io="f16"), [2500, 1, 1100]),
    "k256_v64_bf16_long": (dict(HQ=1, H=2, K=256, V=64, io="bf16"), [1500, 3]),
}


@pytest.mark.parametrize("name", sorted(LONG))
def test_chunk_width_long_sequences(torch, name):
    geo, lens = LONG[name]
    w = workloads.make(name=name, seed=1230 + sorted(LONG).index(name), lengths=lens, **geo)
    print(f"[chunk width long] {name} K={w.K} V={w.V} {w.io} lengths={lens}", flush=True)
    check_chunk(torch, w, name)


CAPTURE = {
    # (geometry, lengths, counts, cap): g and k^ from the first value part, delta from every part
    "k256_v64_f16_g4_cap8": (dict(HQ=1, H=4, K=256, V=64, io="f16"), [70, 5, 0, 130], [8, 5, 3, 2], 8),
    "k96_v320_bf16_cap16": (dict(HQ=1, H=2, K=96, V=320, io="bf16"), [20, 90, 1], [16, 16, 1], 16),
}


@pytest.mark.parametrize("name", sorted(CAPTURE))
def test_chunk_width_capture_against_oracle(torch, name):
    import gated_delta_rule_varlen_amd as gdn

    geo, lens, counts, cap = CAPTURE[name]
    w = workloads.make(name=name, seed=1250 + sorted(CAPTURE).index(name), lengths=lens, **geo)
    counts = np.array(counts, np.int32)
    print(f"[chunk width capture] {name} cap={cap} counts={counts.tolist()}", flush=True)
    kw = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype),
              A_log=dev(w.A_log, "f32"), dt_bias=dev(w.dt_bias, "f32"), state_in=dev(w.state, "f32"), path="chunk")
    qkv, off = dev(w.qkv, w.io), dev_i32(w.offsets)
    o1, s1, used1 = gdn.scan_varlen(qkv, off, **kw)
    o2, s2, caps, used2 = gdn.scan_varlen_capture(
        qkv, off, cap=cap, counts=dev_i32(counts),
        capsule=sentinel((w.B, cap * (w.H + w.HQ * w.K + w.H * w.V)), "f32"), **kw)
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


def test_auto_takes_chunk_at_page_widths(torch):
    """AUTO sends a prefill at K != V (and at padded widths) to the chunked form."""
    for geo in (dict(HQ=1, H=2, K=256, V=64, io="f16"), dict(HQ=1, H=2, K=48, V=80, io="bf16")):
        w = workloads.make(name="auto_width", seed=1260, lengths=[300, 100], **geo)
        out, st, used = gpu_scan(torch, w, "auto", False)
        assert used == "chunk", geo
        o_ref, s_ref = reference(w)
        assert_close(f64(out), o_ref, CHUNK_TOL[w.io], f"auto K={w.K} V={w.V} out")
