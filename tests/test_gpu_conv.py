"""GPU parity of gdn_conv1d_varlen against the oracle, through the C ABI.

Outputs y are compared at the dtype tolerance (1e-4 fp32, 2e-2 half); the carried window is a copy
and must match bit-exactly; malformed offsets must leave every output untouched."""
import numpy as np
import pytest

import cases
import oracle
import workloads
from gpu_util import (TOL, assert_close, bits, channel_subproblem, dev, dev_i32, ensure_built, f64, require_gpu,
                      sentinel)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def gpu_conv(torch, w, x=None, conv_w=None, offsets=None, state=None, inplace=False, dev_status=None):
    import gated_delta_rule_varlen_amd as gdn

    x_d = dev(w.x if x is None else x, w.io)
    y = sentinel(tuple(x_d.shape), w.io)
    st_in = dev(w.conv_state if state is None else state, w.conv_state_dtype)
    st_out = None
    if w.L > 0:
        st_out = st_in if (inplace and st_in is not None) else sentinel((w.B, w.C, w.L), w.conv_state_dtype)
    off = dev_i32(w.offsets if offsets is None else offsets)
    y, st_out = gdn.conv1d_varlen(x_d, dev(w.conv_w if conv_w is None else conv_w, w.io), off,
                                  bias=dev(w.conv_bias, w.io), state_in=st_in, dilation=w.D, silu=w.silu,
                                  state_dtype=getattr(torch, {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}[w.conv_state_dtype]),
                                  y=y, state_out=st_out, dev_status=dev_status)
    torch.cuda.synchronize()
    return y, st_out


def sampled_channels(w, n):
    if w.C <= n:
        return np.arange(w.C)
    rng = np.random.default_rng(7)
    return np.unique(np.concatenate([[0, w.C - 1], rng.choice(w.C, n - 2, replace=False)]))


@pytest.mark.parametrize("name", cases.ALL)
def test_conv_matches_oracle(torch, name):
    w = cases.get(name)
    print(f"[conv parity] {name} B={w.B} N={w.N} C={w.C} W={w.W} D={w.D} io={w.io}", flush=True)
    y, st = gpu_conv(torch, w)
    chans = sampled_channels(w, {"prefill": 384, "long": 256}.get(name, w.C))
    sub = channel_subproblem(w, chans)
    y_ref, st_ref = oracle.conv(sub.pop("x"), sub.pop("w"), w.offsets, **sub)
    yg = f64(y)[:, chans]
    assert np.all(np.isfinite(yg)), "a token row was left unwritten"
    assert np.all(np.isfinite(f64(y))), "a token row was left unwritten"
    assert_close(yg, y_ref, TOL[w.io], f"{name} conv y")
    if w.L > 0:
        assert np.array_equal(f64(st)[:, chans], st_ref), f"{name}: carried window is not an exact copy"


@pytest.mark.parametrize("name", ["tiny_fp32", "edge_fp16", "decode"])
def test_delta_weight_is_exact_identity(torch, name):
    w = cases.get(name)
    wd = np.zeros((w.C, w.W), np.float32)
    wd[:, w.W - 1] = 1.0
    import dataclasses

    w2 = dataclasses.replace(w, conv_bias=None, silu=False)
    y, _ = gpu_conv(torch, w2, conv_w=workloads.to_raw(wd, w.io))
    # exact by value: 0 + (-0) = +0, so a signed zero in x comes back as +0 (the oracle agrees)
    assert np.array_equal(f64(y), workloads.from_raw(w.x, w.io).astype(np.float64))


@pytest.mark.parametrize("name", ["tiny_fp32", "edge_fp16", "decode"])
def test_in_place_window_update_matches_out_of_place(torch, name):
    w = cases.get(name)
    y1, st1 = gpu_conv(torch, w)
    y2, st2 = gpu_conv(torch, w, inplace=True)
    assert np.array_equal(bits(y1), bits(y2))
    assert np.array_equal(bits(st1), bits(st2))


@pytest.mark.parametrize("name", ["tiny_fp32", "edge_fp16"])
def test_malformed_offsets_write_nothing(torch, name):
    w = cases.get(name)
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    gpu_conv(torch, w, dev_status=status)
    assert int(status.item()) == 0
    for case, bad in workloads.malformed_offsets(w.offsets):
        print(f"[conv malformed] {name} {case}", flush=True)
        y, st = gpu_conv(torch, w, offsets=bad, dev_status=status)
        assert int(status.item()) == -9, case
        assert np.all(bits(y) == bits(sentinel(tuple(y.shape), w.io))), case
        assert np.all(bits(st) == bits(sentinel(tuple(st.shape), w.conv_state_dtype))), case


def test_all_sequences_empty_copies_windows(torch):
    w = cases.get("edge_fp16")
    import dataclasses

    w0 = dataclasses.replace(w, N=0, offsets=np.zeros(w.B + 1, np.int32), x=w.x[:0], qkv=w.qkv[:0])
    _, st = gpu_conv(torch, w0)
    assert np.array_equal(bits(st), np.ascontiguousarray(w.conv_state).view(np.int16))


SWEEP = [(W, D, io, sdt) for W in (2, 6, 8) for D in (1, 3) for io, sdt in (("bf16", "f32"), ("f16", "f16"), ("f32", "f32"))]


@pytest.mark.parametrize("W,D,io,sdt", SWEEP)
def test_conv_widths_and_dilations(torch, W, D, io, sdt):
    """Conv widths up to the supported maximum (8) and dilations beyond 1, with window dtypes equal to
    and wider than x: sequences empty, shorter than the window, and long (several body tiles)."""
    lens = [0, 1, 2, 5, 40, 7, 0, 63]
    w = workloads.make(name=f"conv_w{W}_d{D}_{io}", seed=900 + 10 * W + D, lengths=lens, HQ=1, H=1, K=32, V=64,
                       W=W, D=D, io=io, conv_state_dtype=sdt)
    print(f"[conv sweep] W={W} D={D} {io}/{sdt} L={w.L}", flush=True)
    y, st = gpu_conv(torch, w)
    y_ref, st_ref = oracle.conv(w.x, w.conv_w, w.offsets, W=w.W, D=w.D, x_dtype=w.io, bias=w.conv_bias,
                                state_in=w.conv_state, state_dtype=w.conv_state_dtype, silu=w.silu)
    assert_close(f64(y), y_ref, TOL[w.io], "y")
    assert np.array_equal(f64(st), st_ref), "the new window is a copy"
    y2, st2 = gpu_conv(torch, w, inplace=True)
    assert np.array_equal(bits(y2), bits(y)) and np.array_equal(bits(st2), bits(st))


WIDE = [(W, D, io, sdt) for W in (9, 12, 16) for D in (1, 3) for io, sdt in (("bf16", "f32"), ("f16", "f16"), ("f32", "f32"))]


@pytest.mark.parametrize("W,D,io,sdt", WIDE)
def test_conv_wide_widths(torch, W, D, io, sdt):
    """Widths past 8 (the pages' conv has no width limit) run on the per-element form: outputs
    against the oracle, the new window a bit copy, in place bit-identical, with sequences empty,
    shorter than the window (L = (W-1) D up to 45) and long, and an odd channel count."""
    lens = [0, 1, 2, 5, 40, 7, 0, 63, 130]
    w = workloads.make(name=f"conv_wide_w{W}_d{D}_{io}", seed=1300 + 10 * W + D, lengths=lens, HQ=1, H=1, K=32, V=61,
                       W=W, D=D, io=io, conv_state_dtype=sdt)
    print(f"[conv wide] W={W} D={D} {io}/{sdt} L={w.L} C={w.C}", flush=True)
    y, st = gpu_conv(torch, w)
    y_ref, st_ref = oracle.conv(w.x, w.conv_w, w.offsets, W=w.W, D=w.D, x_dtype=w.io, bias=w.conv_bias,
                                state_in=w.conv_state, state_dtype=w.conv_state_dtype, silu=w.silu)
    assert_close(f64(y), y_ref, TOL[w.io], "y")
    assert np.array_equal(f64(st), st_ref), "the new window is a copy"
    y2, st2 = gpu_conv(torch, w, inplace=True)
    assert np.array_equal(bits(y2), bits(y)) and np.array_equal(bits(st2), bits(st))


def test_conv_wide_malformed_offsets_write_nothing(torch):
    w = workloads.make(name="conv_wide_bad", seed=1399, lengths=[3, 0, 9, 4], HQ=1, H=1, K=32, V=64, W=12, D=2,
                       io="bf16", conv_state_dtype="f32")
    for case, bad in workloads.malformed_offsets(w.offsets):
        print(f"[conv wide malformed] {case}", flush=True)
        status = dev_i32(np.array([12345]))
        y, st = gpu_conv(torch, w, offsets=bad, dev_status=status)
        assert int(status.cpu()[0]) == -9
        assert np.all(bits(y) == bits(sentinel(tuple(y.shape), w.io)))
        assert np.all(bits(st) == bits(sentinel(tuple(st.shape), w.conv_state_dtype)))
