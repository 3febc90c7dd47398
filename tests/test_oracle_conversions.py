"""Pins of the oracle's fp16 / bf16 conversions against library conversions.

numpy's float16 cast and torch's bfloat16 cast are both IEEE round-to-nearest-even;
the oracle's bit-level implementations must agree with them on every pattern tried.
"""
import numpy as np
import torch


def _all_f16_patterns():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (h >> 10) & 0x1F
    return h[exp != 31]  # finite only


def test_f16_roundtrip_all_finite_patterns(oracle_mod):
    h = _all_f16_patterns()
    f = oracle_mod.f16_bits_to_f32(h)
    np.testing.assert_array_equal(f, h.view(np.float16).astype(np.float32))
    back = oracle_mod.f32_to_f16_bits(f)
    # -0 and +0 both round-trip to themselves
    np.testing.assert_array_equal(back, h)


def test_f16_midpoints_round_to_even(oracle_mod):
    h = _all_f16_patterns()
    pos = h[(h & 0x8000) == 0]
    pos = pos[pos < 0x7BFF]  # successor must be finite
    lo = pos.view(np.float16).astype(np.float64)
    hi = (pos + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact: 12 significant bits
    assert np.all(mid.astype(np.float64) == (lo + hi) / 2)
    ref = mid.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle_mod.f32_to_f16_bits(mid), ref)
    np.testing.assert_array_equal(oracle_mod.f32_to_f16_bits(-mid), ref | 0x8000)
    # ties go to the even neighbour
    even = np.where((pos & 1) == 0, pos, pos + 1).astype(np.uint16)
    np.testing.assert_array_equal(ref, even)


def test_f16_random_and_strided_fp32(oracle_mod):
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(2_000_000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(1_000_000) * 1e-5).astype(np.float32),  # fp16 subnormal range
        (rng.uniform(-65519, 65519, 500_000)).astype(np.float32),
        np.arange(0, 1 << 32, 4099, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle_mod.f32_to_f16_bits(x), ref)


def test_f16_edges(oracle_mod):
    x = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e30, -1e30, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 6.103515625e-05, 6.1e-05, 1e-40],
                 dtype=np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle_mod.f32_to_f16_bits(x), ref)


def test_bf16_against_torch(oracle_mod):
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(2_000_000).astype(np.float32) * np.float32(10.0),
        np.arange(0, 1 << 32, 8191, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle_mod.f32_to_bf16_bits(x), ref)
    # every bf16 pattern is a fixed point
    b = np.arange(1 << 16, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    fin = np.isfinite(f)
    np.testing.assert_array_equal(oracle_mod.f32_to_bf16_bits(f[fin]), b[fin].astype(np.uint16))
