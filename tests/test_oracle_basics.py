"""Pins for the oracle's element decoders and offsets check (CPU only)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_f16_decoder_matches_numpy_on_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.decode(bits, oracle.F16)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_bf16_decoder_matches_torch_on_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = oracle.decode(bits, oracle.BF16)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_f32_decoder_is_identity():
    x = np.random.default_rng(0).standard_normal(257).astype(np.float32)
    assert np.array_equal(oracle.decode(x, oracle.F32), x.astype(np.float64))


@pytest.mark.parametrize(
    "off,B,N,ok",
    [
        ([0, 37, 64], 2, 64, True),
        ([0, 0, 0], 2, 0, True),  # all sequences empty
        ([0, 0, 5, 5], 3, 5, True),  # zero-length first and last
        ([1, 37, 64], 2, 64, False),  # first entry not zero
        ([0, 37, 63], 2, 64, False),  # last entry below N
        ([0, 37, 65], 2, 64, False),  # last entry above N
        ([0, 40, 30, 64], 3, 64, False),  # interior decrease
        ([0, -1, 64], 2, 64, False),  # negative entry
        ([0, 70, 64], 2, 64, False),  # entry above N (and a decrease)
        ([0], 0, 0, False),  # B must be at least 1
    ],
)
def test_offsets_truth_table(off, B, N, ok):
    assert oracle.offsets_valid(np.array(off, np.int32), B, N) is ok
