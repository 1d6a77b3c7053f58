"""Seeded synthetic inputs for the varlen gated delta-rule hot path.

Shared by the tests, the benchmark and the smoke check; used by both the HIP path and the oracle,
so it holds none of the method's arithmetic: only random draws (numpy ``default_rng``), dtype
casts with round-to-nearest-even, and offsets built from drawn lengths.

Half-precision tensors are stored as raw ``uint16`` bit patterns (bf16 or IEEE f16); fp32 tensors
as ``float32``.  The packed token row is ``[q: HQ*K | k: HQ*K | v: H*V]`` and the conv runs over
all ``C = 2*HQ*K + H*V`` channels of it.

Draw order inside :func:`make` (fixed, so a seed names one input set):
  lengths -> x -> conv weight -> conv bias -> conv window -> scan qkv (only when drawn separately)
  -> decay input a -> rate input b -> A_log -> dt_bias -> recurrent state.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

IO_DTYPES = ("f32", "bf16", "f16")


def to_raw(a: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float data to the storage of ``dtype`` with round-to-nearest-even."""
    a = np.asarray(a, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(a)
    if dtype == "f16":
        return np.ascontiguousarray(a.astype(np.float16).view(np.uint16))
    if dtype == "bf16":
        u = a.view(np.uint32).astype(np.uint64)
        r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return np.ascontiguousarray(r.astype(np.uint16))
    raise ValueError(dtype)


def from_raw(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Storage -> float32 values (exact for every dtype used here)."""
    if dtype == "f32":
        return np.asarray(raw, np.float32)
    if dtype == "f16":
        return np.asarray(raw, np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(raw, np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    N: int
    HQ: int
    H: int
    K: int
    V: int
    W: int
    D: int
    io: str  # dtype of x, conv weight/bias, qkv and outputs
    gate_dtype: str  # dtype of a and b
    conv_state_dtype: str
    l2norm: bool
    softplus: bool
    sigmoid: bool
    silu: bool
    offsets: np.ndarray  # int32 [B+1]
    x: np.ndarray  # [N, C] conv input
    conv_w: np.ndarray  # [C, W]
    conv_bias: Optional[np.ndarray]  # [C]
    conv_state: Optional[np.ndarray]  # [B, C, L]
    qkv: np.ndarray  # [N, C] scan input
    a: Optional[np.ndarray]  # [N, H]
    b: Optional[np.ndarray]  # [N, H]
    A_log: Optional[np.ndarray]  # [H] f32
    dt_bias: Optional[np.ndarray]  # [H] f32
    state: Optional[np.ndarray]  # [B, H, V, K] f32
    scale: float = 0.0  # 0 selects 1/sqrt(K); any other value is applied

    @property
    def C(self) -> int:
        return 2 * self.HQ * self.K + self.H * self.V

    @property
    def L(self) -> int:
        return (self.W - 1) * self.D

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets)


def offsets_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, np.int64)
    off[1:] = np.cumsum(np.asarray(lengths, np.int64))
    return off.astype(np.int32)


def make(*, name: str, seed: int, lengths: Sequence[int] | None = None, length_range=None, B: int = 1,
         force_zero: Sequence[int] = (), HQ: int, H: int, K: int, V: int, W: int = 4, D: int = 1,
         io: str = "bf16", gate_dtype: str | None = None, conv_state_dtype: str | None = None,
         l2norm: bool = True, softplus: bool = True, sigmoid: bool = True, silu: bool = True,
         has_bias: bool = True, conv_w_std: float = 0.5, conv_bias_std: float = 0.5,
         conv_state_std: float | None = 1.0, state_std: float | None = 0.1,
         A_log_range=(0.0, math.log(16.0)), dt_bias_std: float = 0.5, decay_range=None,
         beta_range=None, unit_k_scan: bool = False, has_decay: bool = True, has_beta: bool = True) -> Workload:
    """Draw one synthetic workload.  ``conv_state_std``/``state_std`` of None give zero (absent)
    initial states; ``decay_range``/``beta_range`` draw raw U[lo,hi] gate inputs instead of N(0,1)
    logits; ``unit_k_scan`` draws the scan's qkv separately with q ~ N(0, 1/K), unit-norm k rows and
    v ~ N(0, 1) (for runs without q/k normalisation)."""
    rng = np.random.default_rng(seed)
    gate_dtype = gate_dtype or io
    conv_state_dtype = conv_state_dtype or io
    if lengths is None:
        lo, hi = length_range
        lengths = rng.integers(lo, hi + 1, size=B)
    lengths = np.asarray(lengths, np.int64).copy()
    for i in force_zero:
        lengths[i] = 0
    B = len(lengths)
    offsets = offsets_from_lengths(lengths)
    N = int(offsets[-1])
    C = 2 * HQ * K + H * V
    L = (W - 1) * D

    x = to_raw(rng.standard_normal((N, C), dtype=np.float32), io)
    conv_w = to_raw(rng.standard_normal((C, W), dtype=np.float32) * conv_w_std, io)
    conv_bias = to_raw(rng.standard_normal(C, dtype=np.float32) * conv_bias_std, io) if has_bias else None
    conv_state = None
    if conv_state_std is not None and L > 0:
        conv_state = to_raw(rng.standard_normal((B, C, L), dtype=np.float32) * conv_state_std, conv_state_dtype)

    if unit_k_scan:
        q = rng.standard_normal((N, HQ, K), dtype=np.float32) / np.float32(math.sqrt(K))
        k = rng.standard_normal((N, HQ, K), dtype=np.float32)
        k /= np.linalg.norm(k, axis=-1, keepdims=True).astype(np.float32) + np.float32(1e-30)
        v = rng.standard_normal((N, H * V), dtype=np.float32)
        qkv = to_raw(np.concatenate([q.reshape(N, -1), k.reshape(N, -1), v], axis=1), io)
    else:
        qkv = x

    a = b = None
    if has_decay:
        if decay_range is None:
            a = rng.standard_normal((N, H), dtype=np.float32)
        else:
            a = rng.uniform(decay_range[0], decay_range[1], size=(N, H)).astype(np.float32)
        a = to_raw(a, gate_dtype)
    if has_beta:
        if beta_range is None:
            b = rng.standard_normal((N, H), dtype=np.float32)
        else:
            b = rng.uniform(beta_range[0], beta_range[1], size=(N, H)).astype(np.float32)
        b = to_raw(b, gate_dtype)
    A_log = dt_bias = None
    if softplus:
        A_log = rng.uniform(A_log_range[0], A_log_range[1], size=H).astype(np.float32)
        dt_bias = (rng.standard_normal(H, dtype=np.float32) * dt_bias_std).astype(np.float32)
    state = None
    if state_std is not None:
        state = (rng.standard_normal((B, H, V, K), dtype=np.float32) * np.float32(state_std)).astype(np.float32)

    return Workload(name=name, B=B, N=N, HQ=HQ, H=H, K=K, V=V, W=W, D=D, io=io, gate_dtype=gate_dtype,
                    conv_state_dtype=conv_state_dtype, l2norm=l2norm, softplus=softplus, sigmoid=sigmoid,
                    silu=silu, offsets=offsets, x=x, conv_w=conv_w, conv_bias=conv_bias,
                    conv_state=conv_state, qkv=qkv, a=a, b=b, A_log=A_log, dt_bias=dt_bias, state=state)


# ---- the five named workloads ------------------------------------------------------------------

def tiny_fp32(seed: int = 101) -> Workload:
    """B=2 sequences of 37 and 27 tokens, HQ=H=2, K=V=32, fp32, all activations, zero states."""
    return make(name="tiny_fp32", seed=seed, lengths=[37, 27], HQ=2, H=2, K=32, V=32, W=4, D=1, io="f32",
                conv_state_std=None, state_std=None, dt_bias_std=0.0)


def decode_step(seed: int = 102) -> Workload:
    """B=256 sequences x 1 token, HQ=16, H=32, K=V=128, bf16, fp32 state and conv window."""
    return make(name="decode_b256_h32_k128", seed=seed, lengths=[1] * 256, HQ=16, H=32, K=128, V=128, W=4,
                D=1, io="bf16", conv_state_dtype="f32", conv_state_std=1.0, state_std=0.1)


def varlen_prefill(seed: int = 103) -> Workload:
    """B=8 sequences, lengths ~ U[512, 4096], HQ=16, H=32, K=V=128, bf16."""
    return make(name="prefill_b8_u512_4096_h32_k128", seed=seed, B=8, length_range=(512, 4096), HQ=16, H=32,
                K=128, V=128, W=4, D=1, io="bf16", conv_state_dtype="f32", conv_state_std=1.0, state_std=0.1)


def long_single(seed: int = 104, N: int = 65536) -> Workload:
    """B=1, N=65536 tokens, HQ=H=16, K=V=128, bf16, zero initial states."""
    return make(name=f"long_n{N}_h16_k128", seed=seed, lengths=[N], HQ=16, H=16, K=128, V=128, W=4, D=1,
                io="bf16", conv_state_dtype="f32", conv_state_std=None, state_std=None)


def edge_fp16(seed: int = 105) -> Workload:
    """B=64 ragged lengths ~ U[0, 300] (zeros forced at 0, 31, 63), HQ=4, H=16, K=256, V=64, fp16;
    no L2 norm, raw log-decay ~ U[-1, 0], raw beta ~ U[0, 1]; conv W=3, D=2, no bias, no SiLU."""
    return make(name="edge_fp16_b64_k256_v64", seed=seed, B=64, length_range=(0, 300), force_zero=(0, 31, 63),
                HQ=4, H=16, K=256, V=64, W=3, D=2, io="f16", conv_state_dtype="f16", l2norm=False,
                softplus=False, sigmoid=False, silu=False, has_bias=False, conv_state_std=1.0, state_std=0.1,
                decay_range=(-1.0, 0.0), beta_range=(0.0, 1.0), unit_k_scan=True)


def spec_verify(seed: int = 106) -> Workload:
    """A speculative-decoding verification step: B=256 sequences x 5 tokens (the last accepted token
    and 4 drafts), HQ=16, H=32, K=V=128, bf16, fp32 state and conv window."""
    return make(name="verify_b256_t5_h32_k128", seed=seed, lengths=[5] * 256, HQ=16, H=32, K=128, V=128, W=4,
                D=1, io="bf16", conv_state_dtype="f32", conv_state_std=1.0, state_std=0.1)


def mixed_batch(seed: int = 107) -> Workload:
    """A serving batch that mixes decode and prefill: 255 sequences x 1 token and one 4096-token
    sequence (N = 4351), HQ=16, H=32, K=V=128, bf16, fp32 state and conv window."""
    return make(name="mixed_b256_255x1_1x4096_h32_k128", seed=seed, lengths=[1] * 255 + [4096], HQ=16, H=32,
                K=128, V=128, W=4, D=1, io="bf16", conv_state_dtype="f32", conv_state_std=1.0, state_std=0.1)


NAMED = {
    "tiny_fp32": tiny_fp32,
    "decode": decode_step,
    "prefill": varlen_prefill,
    "long": long_single,
    "edge_fp16": edge_fp16,
    "verify": spec_verify,
    "mixed": mixed_batch,
}

# Offsets patterns that every entry point must reject by writing nothing.
def malformed_offsets(offsets: np.ndarray) -> list[tuple[str, np.ndarray]]:
    off = np.asarray(offsets, np.int32)
    B = off.size - 1
    N = int(off[-1])
    cases = []
    o = off.copy(); o[0] = 1; cases.append(("first_nonzero", o))
    o = off.copy(); o[-1] = N + 1; cases.append(("last_above_n", o))
    o = off.copy(); o[-1] = N - 1; cases.append(("last_below_n", o))
    if B >= 3:
        o = off.copy(); i = B // 2; o[i] = o[i + 1] + 1; cases.append(("interior_decrease", o))
    o = off.copy(); o[min(1, B - 1)] = -1
    if B >= 2:
        cases.append(("negative_entry", o))
    o = off.copy(); o[min(1, B - 1)] = N + 5
    if B >= 2:
        cases.append(("entry_above_n", o))
    return cases
