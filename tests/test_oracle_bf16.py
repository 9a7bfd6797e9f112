"""Pins the two independent bf16 roundings: the oracle's (fp64 -> bf16, value
space) and the input generator's (fp32 -> bf16, bit arithmetic)."""

import numpy as np
import torch

from oracle import bf16_bits_to_f64, f64_to_bf16_bits
from synth import f32_to_bf16_bits


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    keep = np.isfinite(v)
    return bits[keep], v[keep]


def test_decode_matches_ieee_layout():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x0001 = smallest subnormal 2**-133, 0x7F7F = max finite.
    v = bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16))
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0 ** -133
    assert v[3] == (2 - 2 ** -7) * 2.0 ** 127 and v[4] == 0.0 and np.signbit(v[4])


def test_identity_on_every_finite_bf16():
    bits, v = _all_finite_bf16()
    back = f64_to_bf16_bits(v)
    # -0.0 and 0.0 keep their sign bit
    assert np.array_equal(back, bits)


def test_midpoints_round_to_even_and_off_midpoints_to_nearest():
    bits, v = _all_finite_bf16()
    pos = (bits < 0x7F7F) & (bits >= 0x0000) & (v >= 0)
    lo_bits = bits[pos]
    lo = v[pos]
    hi_bits = (lo_bits + 1).astype(np.uint16)
    hi = bf16_bits_to_f64(hi_bits)
    mid = (lo + hi) / 2                      # exact in fp64
    got = f64_to_bf16_bits(mid)
    even = np.where(lo_bits % 2 == 0, lo_bits, hi_bits)
    assert np.array_equal(got, even)
    gap = hi - lo
    assert np.array_equal(f64_to_bf16_bits(mid - gap / 8), lo_bits)
    assert np.array_equal(f64_to_bf16_bits(mid + gap / 8), hi_bits)
    assert np.array_equal(f64_to_bf16_bits(-(mid + gap / 8)), (hi_bits | 0x8000).astype(np.uint16))


def test_overflow_to_inf():
    top = bf16_bits_to_f64(np.array([0x7F7F], dtype=np.uint16))[0]
    ulp = 2.0 ** (127 - 7)
    assert f64_to_bf16_bits(np.array([top + ulp / 4]))[0] == 0x7F7F
    assert f64_to_bf16_bits(np.array([top + ulp / 2]))[0] == 0x7F80      # tie goes to even -> inf
    assert f64_to_bf16_bits(np.array([-1e300]))[0] == 0xFF80


def test_generator_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(10000) * 1e-39).astype(np.float32),       # fp32 subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, np.inf, -np.inf], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_generator_and_oracle_roundings_agree():
    # fp32 -> fp64 is exact, so both must give the same RNE bf16 of the same value.
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    assert np.array_equal(f32_to_bf16_bits(x), f64_to_bf16_bits(x.astype(np.float64)))
