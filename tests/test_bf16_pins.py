"""Pins of the bfloat16 conversions both sides read the cache through.

The oracle's decoder (bit patterns -> exact values) and the input
generator's encoder (fp32 -> bfloat16, round to nearest, ties to even) are
checked against torch's own bfloat16 conversion on the CPU, an independent
implementation of the same format ("How to use it" on the CompKV page: the
KV cache is stored in BF16).
"""
import numpy as np
import pytest

from block_sparse_kv_stats_amd import synth
from oracle import compkv as ok

torch = pytest.importorskip("torch")


def torch_decode(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def torch_encode(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_decode_every_bit_pattern():
    """All 65536 patterns: the same value (NaN patterns decode to NaN), and
    the same sign of zero."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = ok.decode_bf16(bits)
    ref = torch_decode(bits)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127  # exponent all ones, nonzero mantissa, both signs
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_known_values():
    """A few patterns whose values follow from the format by hand."""
    cases = {0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3F00: 0.5, 0x3FC0: 1.5,
             0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x7F80: np.inf}
    got = ok.decode_bf16(np.array(list(cases), dtype=np.uint16))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))


def _encoder_inputs():
    rng = np.random.default_rng(11)
    x = [rng.standard_normal(20000).astype(np.float32),
         (rng.standard_normal(20000) * 1e-39).astype(np.float32),      # subnormals
         (rng.standard_normal(5000) * 3e38).astype(np.float32),        # near the top of the range
         np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max,
                   -np.finfo(np.float32).max, np.finfo(np.float32).tiny], dtype=np.float32)]
    # exact halfway cases: low 16 bits 0x8000, with even and odd kept mantissa
    hi = rng.integers(0, 0x7F7F, 4000, dtype=np.uint32)
    x.append(((hi << 16) | 0x8000).view(np.float32))
    x.append(((hi << 16) | 0x8000 | 0x80000000).view(np.float32))
    # one above and one below halfway
    x.append(((hi << 16) | 0x8001).view(np.float32))
    x.append(((hi << 16) | 0x7FFF).view(np.float32))
    return np.concatenate(x).astype(np.float32)


def test_encoder_matches_torch_round_to_nearest_even():
    x = _encoder_inputs()
    np.testing.assert_array_equal(synth.bf16_bits(x), torch_encode(x))


def test_encoder_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0);
    # 1 + 3*2^-8 lies between 1 + 2^-7 (odd) and 1 + 2^-6: rounds up to the even one
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], dtype=np.float32)
    np.testing.assert_array_equal(synth.bf16_bits(x), np.array([0x3F80, 0x3F82], dtype=np.uint16))


def test_round_trip_is_exact_on_representable_values():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = ok.decode_bf16(bits)
    fin = np.isfinite(vals)
    np.testing.assert_array_equal(synth.bf16_bits(vals[fin].astype(np.float32)), bits[fin])
