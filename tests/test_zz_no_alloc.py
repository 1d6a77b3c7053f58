"""gdn_scan_varlen_noalloc through the C ABI: the same results, bit for bit, as gdn_scan_varlen with a
caller-allocated workspace, on two calls in a row (the second smaller, so it runs on what the first
left in the library's device array), for the chunked path that uses the array and for the paths that
need no workspace; and a chunked call whose workspace exceeds the array is refused."""
import numpy as np
import pytest

import workloads
from gpu_util import bits, dev, dev_i32, ensure_built, require_gpu, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


def _inputs(w):
    return dict(qkv=dev(w.qkv, w.io), a=dev(w.a, w.gate_dtype), b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"),
                dt_bias=dev(w.dt_bias, "f32"), state_in=dev(w.state, "f32"), offsets=dev_i32(w.offsets))


def _run(torch, gdn, w, path, noalloc):
    x = _inputs(w)
    out = sentinel((w.N, w.H, w.V), w.io)
    st = sentinel((w.B, w.H, w.V, w.K), "f32")
    kw = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=x["a"], b=x["b"], A_log=x["A_log"], dt_bias=x["dt_bias"],
              state_in=x["state_in"], l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid, path=path, out=out,
              state_out=st)
    if noalloc:
        out, st, used = gdn.scan_varlen_noalloc(x["qkv"], x["offsets"], **kw)
    else:
        out, st, used = gdn.scan_varlen(x["qkv"], x["offsets"], **kw)
    torch.cuda.synchronize()
    return bits(out), bits(st), used


# (name, seed, lengths, HQ, H, K, V, io, path): each pair runs the larger batch first
CASES = [
    ("chunk", 11, [300, 0, 517, 129], 2, 4, 64, 64, "bf16", "chunk"),
    ("chunk", 12, [70, 5], 2, 4, 64, 64, "bf16", "chunk"),
    ("auto_prefill", 13, [400, 260, 333], 2, 2, 128, 128, "f16", "auto"),
    ("auto_prefill", 14, [90, 64], 2, 2, 128, 128, "f16", "auto"),
    ("seq", 15, [50, 0, 31], 1, 2, 32, 32, "f32", "seq"),
    ("seq", 16, [9], 1, 2, 32, 32, "f32", "seq"),
    ("decode", 17, [1] * 16, 2, 4, 64, 64, "bf16", "auto"),
    ("decode", 18, [1] * 3, 2, 4, 64, 64, "bf16", "auto"),
]


@pytest.mark.parametrize("pair", [0, 1, 2, 3])
def test_noalloc_matches_allocating_call_twice(torch, pair):
    import gated_delta_rule_varlen_amd as gdn

    for name, seed, lengths, HQ, H, K, V, io, path in CASES[2 * pair:2 * pair + 2]:
        w = workloads.make(name=name, seed=seed, lengths=lengths, HQ=HQ, H=H, K=K, V=V, io=io)
        print(f"[noalloc] {name} seed={seed} lengths={lengths} K={K} V={V} io={io} path={path}", flush=True)
        o_ref, s_ref, used_ref = _run(torch, gdn, w, path, noalloc=False)
        o, s, used = _run(torch, gdn, w, path, noalloc=True)
        assert used == used_ref, (used, used_ref)
        if name.startswith("chunk") or name.startswith("auto"):
            assert used == "chunk"
        assert np.array_equal(o, o_ref), "output differs from gdn_scan_varlen"
        assert np.array_equal(s, s_ref), "final state differs from gdn_scan_varlen"


def test_noalloc_refuses_a_workspace_beyond_the_array(torch):
    import gated_delta_rule_varlen_amd as gdn
    from gated_delta_rule_varlen_amd import _abi

    # a chunked call whose workspace exceeds the array: refused on the host, nothing launched
    N, HQ, H, K, V = 1 << 16, 32, 32, 128, 128
    qkv = torch.empty((N, 2 * HQ * K + H * V), dtype=torch.bfloat16, device="cuda")
    need = gdn.scan_workspace_bytes(qkv, 1, HQ=HQ, H=H, K=K, V=V, path="chunk")
    assert need > _abi.NOALLOC_SCRATCH_BYTES
    off = dev_i32(np.array([0, N], np.int32))
    a = torch.zeros((N, H), dtype=torch.bfloat16, device="cuda")
    alog = torch.zeros(H, dtype=torch.float32, device="cuda")
    out = torch.empty((N, H, V), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((1, H, V, K), dtype=torch.float32, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.scan_varlen_noalloc(qkv, off, HQ=HQ, H=H, K=K, V=V, a=a, A_log=alog, dt_bias=alog, path="chunk", out=out,
                                state_out=st)
    assert e.value.status == _abi.ERR_WORKSPACE
