"""Pin of the oracle's bf16 rounding against torch's fp32 -> bfloat16 cast."""

import numpy as np
import torch

import oracle as O


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_random_values_match_torch():
    rng = np.random.default_rng(0)
    f = (rng.standard_normal(200000) * np.exp(rng.uniform(-60, 60, 200000))).astype(np.float32)
    assert np.array_equal(O.bf16_bits_from_f32(f), _torch_bf16_bits(f))


def test_exact_ties_round_to_even():
    rng = np.random.default_rng(1)
    hi = rng.integers(0, 0x7F7F, 5000, dtype=np.uint32) << 16
    ties = (hi | 0x8000).view(np.float32)
    assert np.array_equal(O.bf16_bits_from_f32(ties), _torch_bf16_bits(ties))
    # explicit: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> 1 (even)
    assert O.bf16_bits_from_f32(np.float32([1 + 2 ** -8]))[0] == 0x3F80
    assert O.bf16_bits_from_f32(np.float32([1 + 3 * 2 ** -8]))[0] == 0x3F82


def test_special_values():
    f = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3.4e38, -3.4e38,
                  1.17549435e-38, 3.3961775e38], dtype=np.float32)
    assert np.array_equal(O.bf16_bits_from_f32(f), _torch_bf16_bits(f))
    nan = O.bf16_bits_from_f32(np.array([np.nan], dtype=np.float32))
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0


def test_bf16_to_f64_is_exact():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.f64_from_bf16_bits(bits), ref)
