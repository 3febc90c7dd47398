"""Pins of the oracle's Walsh-Hadamard transform and fp32 tree sum.

Walsh-Hadamard: TurboQuant on Quantized Models (topic list) and Statistical Inference ...
Inspired by TurboQuant (scheme KQV) name the transform; Dual-QK sec. 1 states that a
paired query/key transform preserves q.k, which for the orthogonal-up-to-scale Hadamard
matrix reads (Hq).(Hk)/d = q.k.
"""
import math

import numpy as np
import pytest
import scipy.linalg


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_equals_sylvester_matrix_exactly(oracle_mod, d):
    rng = np.random.default_rng(d)
    H = scipy.linalg.hadamard(d).astype(np.int64)
    x = rng.integers(-1000, 1000, size=(20, d))
    ref = x @ H.T  # small integers: exact in fp32
    got32 = oracle_mod.fwht_f32(x.astype(np.float32))
    got64 = oracle_mod.fwht_f64(x.astype(np.float64))
    np.testing.assert_array_equal(got32.astype(np.int64), ref)
    np.testing.assert_array_equal(got64.astype(np.int64), ref)


def _fwht_recursive_f32(x):
    """H_{2n} = [[H_n, H_n], [H_n, -H_n]] evaluated recursively in numpy fp32."""
    n = x.shape[-1]
    if n == 1:
        return x.copy()
    lo = _fwht_recursive_f32(x[..., : n // 2])
    hi = _fwht_recursive_f32(x[..., n // 2:])
    return np.concatenate([lo + hi, lo - hi], axis=-1).astype(np.float32)


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_f32_bit_identical_to_recursive_definition(oracle_mod, d):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((500, d)).astype(np.float32)
    np.testing.assert_array_equal(oracle_mod.fwht_f32(x), _fwht_recursive_f32(x))


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_involution_parseval_and_dot_preservation(oracle_mod, d):
    rng = np.random.default_rng(11)
    q = rng.standard_normal((50, d))
    k = rng.standard_normal((50, d)) * 3.0
    hq, hk = oracle_mod.fwht_f64(q), oracle_mod.fwht_f64(k)
    np.testing.assert_allclose(oracle_mod.fwht_f64(hq), d * q, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose((hq * hq).sum(1), d * (q * q).sum(1), rtol=1e-12)
    np.testing.assert_allclose((hq * hk).sum(1) / d, (q * k).sum(1), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("n", [2, 16, 64, 128])
def test_tree_sum_matches_xor_butterfly_and_fsum(oracle_mod, n):
    rng = np.random.default_rng(n)
    for _ in range(200):
        a = (rng.standard_normal(n) * rng.uniform(0.1, 100)).astype(np.float32) ** 2
        got = oracle_mod.tree_sum_f32(a)
        # xor butterfly over "lanes": v_i <- v_i + v_{i^h}, h = n/2 .. 1; lane 0 holds the tree
        v = a.copy()
        idx = np.arange(n)
        h = n // 2
        while h >= 1:
            v = (v + v[idx ^ h]).astype(np.float32)
            h //= 2
        assert np.all(v == v[0])
        assert got == v[0]
        exact = math.fsum(float(t) for t in a)
        assert abs(float(got) - exact) <= 1e-6 * exact
