"""GPU parity of gdn_prepare_qk_gates against the oracle, through the C ABI (fp32 outputs, 1e-4)."""
import numpy as np
import pytest

import cases
import oracle
from gpu_util import PREP_TOL, assert_close, dev, ensure_built, f64, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    ensure_built()
    return require_gpu()


@pytest.mark.parametrize("name", cases.ALL)
def test_prepare_matches_oracle(torch, name):
    import gated_delta_rule_varlen_amd as gdn

    w = cases.get(name)
    print(f"[prepare parity] {name} N={w.N} HQ={w.HQ} H={w.H} K={w.K} io={w.io}", flush=True)
    qk, gb = gdn.prepare_qk_gates(dev(w.qkv, w.io), HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=dev(w.a, w.gate_dtype),
                                  b=dev(w.b, w.gate_dtype), A_log=dev(w.A_log, "f32"), dt_bias=dev(w.dt_bias, "f32"),
                                  l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid)
    torch.cuda.synchronize()
    # the prepare is token-local: compare a token sample that spans the packed range
    rng = np.random.default_rng(3)
    toks = np.arange(w.N) if w.N <= 4096 else np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 2000, False)]))
    qk_ref, gb_ref = oracle.prepare(np.ascontiguousarray(w.qkv[toks]), HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io,
                                    gate_dtype=w.gate_dtype,
                                    a=None if w.a is None else np.ascontiguousarray(w.a[toks]),
                                    b=None if w.b is None else np.ascontiguousarray(w.b[toks]), A_log=w.A_log,
                                    dt_bias=w.dt_bias, l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid)
    qk_g, gb_g = f64(qk)[:, toks], f64(gb)[:, toks]
    for plane, nm in enumerate("qk"):
        assert_close(qk_g[plane], qk_ref[plane], PREP_TOL, f"{name} prepare {nm}-hat")
    assert_close(gb_g[0], gb_ref[0], PREP_TOL, f"{name} prepare g")
    assert_close(gb_g[1], gb_ref[1], PREP_TOL, f"{name} prepare beta")
    # elementwise on the gates too: small decays must not lose relative accuracy
    big = gb_ref[0] > 1e-30
    np.testing.assert_allclose(gb_g[0][big], gb_ref[0][big], rtol=2e-4)
