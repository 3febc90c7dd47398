"""Pins of the oracle's KQV value format.

Statistical Inference and Quality Measures of KV Cache Quantisations Inspired by TurboQuant,
"Quantisierungsschemata": KQV rotates values with a Walsh-Hadamard transform and stores them
with (n-1)-bit scalar MSE codes plus a 1-bit QJL sketch of the residual, whose estimator is
unbiased with variance (pi/2) ||r||^2 / d ("Theoretischer Beweis ..."); TurboQuant on
Quantized Models (abstract): the sketch matrix is a structured Hadamard transform (SRHT-QJL).
Readings: n = 4 (3-bit codes of the 8-level N(0,1) Lloyd-Max codebook on the rotated value
scaled by its RMS, as for keys), S = H D with the caller's random sign diagonal D, estimator
r^ = sqrt(pi/2) / d * ||r|| * S^T sign(S r), a zero coordinate of S r counting as +.
"""
import os

import numpy as np
import pytest
import scipy.linalg

import format_ref as fr

GOLD = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian_8.txt")


def _signs(rng, d):
    return rng.integers(0, 2 ** 32, size=d // 32, dtype=np.uint64).astype(np.uint32)


def _cache(oracle_mod, d=64, cap=256, signs=None, units=1, ns=0, nr=0):
    g = oracle_mod.Geometry(batch=units, n_kv_heads=1, head_dim=d, capacity=cap, n_sink=ns, k_format=0,
                            v_format=oracle_mod.V_KQV, n_recent=nr)
    return oracle_mod.OracleCache(g, qjl_signs=signs)


def _dvec(signs, d):
    return np.array([-1.0 if (signs[i // 32] >> (i % 32)) & 1 else 1.0 for i in range(d)])


def test_three_bit_codebook_is_max_table(oracle_mod):
    rows = [list(map(float, ln.split()[1:])) for ln in open(GOLD) if ln[0].isdigit()]
    xs, ys = np.array([r[0] for r in rows]), np.array([r[1] for r in rows])
    c, t = oracle_mod.codebook_f32(8)
    np.testing.assert_allclose(c[4:], ys, atol=6e-4)
    np.testing.assert_allclose(t[3:], xs, atol=6e-4)
    np.testing.assert_array_equal(c[:4], -c[4:][::-1])


def _decode_ref(oc, d, T):
    """Second reader: numpy bit arithmetic and explicit matrices, S = H diag(D)."""
    H = scipy.linalg.hadamard(d).astype(np.float64)
    Dm = np.diag(_dvec(oc.qjl, d))
    nib = fr.value_codes(oc.v_codes[0], d, T)
    sz = oc.v_sz[0, 0, :T]
    rho, gam = fr.f16(sz & 0xFFFF), fr.f16(sz >> 16)
    yhat = rho[:, None] * oc.vcent.astype(np.float64)[nib & 7]
    sig = np.where(nib & 8, -1.0, 1.0)
    S = H @ Dm
    rhat = np.sqrt(np.pi / 2) / d * gam[:, None] * (sig @ S)  # rows: S^T sign
    return (yhat + rhat) @ H.T / d, yhat, rho, gam, S


@pytest.mark.parametrize("d", [64, 128])
def test_codes_sketch_and_decode(oracle_mod, d):
    """Codes are the nearest centroid of y / rho (y = H v), the sketch bits are the signs of
    S r with r = y - rho cent[code], gamma = ||r||, and the decode is
    H^T (y^ + sqrt(pi/2)/d gamma S^T sign(S r)) / d: checked against explicit matrices."""
    rng = np.random.default_rng(800 + d)
    T = 300
    signs = _signs(rng, d)
    oc = _cache(oracle_mod, d=d, cap=512, signs=signs)
    v = (rng.standard_normal((1, T, d)) * rng.uniform(0.1, 4, (1, T, 1))).astype(np.float32)
    oc.append(rng.standard_normal((1, T, d)).astype(np.float32), v)
    _, vh = oc.dequant(0)
    ref, yhat, rho, gam, S = _decode_ref(oc, d, T)
    np.testing.assert_allclose(vh, ref, rtol=0, atol=1e-9 * np.abs(ref).max())
    H = scipy.linalg.hadamard(d).astype(np.float64)
    y = v[0].astype(np.float64) @ H.T
    z = y / rho[:, None]
    cent = oc.vcent.astype(np.float64)
    dist = np.abs(z[:, :, None] - cent[None, None, :])
    best = dist.argmin(-1)
    nib = fr.value_codes(oc.v_codes[0], d, T)
    clear = np.sort(dist, -1)[:, :, 1] - np.sort(dist, -1)[:, :, 0] > 1e-4
    assert np.array_equal((nib & 7)[clear], best[clear])
    np.testing.assert_allclose(rho, np.sqrt((y ** 2).mean(1)), rtol=1e-3)
    r = y - yhat
    np.testing.assert_allclose(gam, np.linalg.norm(r, axis=1), rtol=1e-3, atol=1e-6)
    sr = r @ S.T
    clear = np.abs(sr) > 1e-3 * np.linalg.norm(r, axis=1, keepdims=True)
    assert np.array_equal(((nib & 8) > 0)[clear], (sr < 0)[clear])


def test_qjl_estimator_is_unbiased_with_the_stated_variance(oracle_mod):
    """Over random sign diagonals D, the error <q, v^ - v> of a fixed value averages to 0 and
    its variance stays within (pi/2) ||r||^2 ||q||^2 / d (r the residual in the rotated
    coordinates, q unit-norm in the value's coordinates); without the sketch the error is
    the fixed -<q, r>-like bias."""
    rng = np.random.default_rng(810)
    d, N = 64, 3000
    v = rng.standard_normal((1, 1, d)).astype(np.float32)
    q = rng.standard_normal(d)
    q /= np.linalg.norm(q)
    errs, rn = [], None
    for _ in range(N):
        oc = _cache(oracle_mod, d=d, signs=_signs(rng, d))
        oc.append(v, v)
        _, vh = oc.dequant(0)
        errs.append(float(q @ (vh[0] - v[0, 0])))
        if rn is None:
            _, yhat, _, _, _ = _decode_ref(oc, d, 1)
            H = scipy.linalg.hadamard(d).astype(np.float64)
            r = v[0, 0].astype(np.float64) @ H.T - yhat[0]
            rn = np.linalg.norm(r)
            bias = float(q @ (yhat[0] @ H.T / d - v[0, 0]))  # codes alone
    errs = np.array(errs)
    # the value error is (H^T r^ - H^T r) / d: in unit-norm terms ||r|| / sqrt(d)
    var_bound = np.pi / 2 * (rn / np.sqrt(d)) ** 2 / d
    assert errs.var() <= 1.2 * var_bound
    assert abs(errs.mean()) <= 4 * np.sqrt(var_bound / N)
    assert abs(bias) > 6 * np.sqrt(var_bound / N)  # the sketch removes a bias the codes have


def test_attention_over_kqv_values_and_bf16_positions(oracle_mod):
    """Attention output = softmax-weighted sum of the decoded values (second reader), with
    sinks and a recent window kept in BF16 in the values' own coordinates."""
    rng = np.random.default_rng(820)
    d, T, G = 64, 200, 2
    oc = _cache(oracle_mod, d=d, cap=256, signs=_signs(rng, d), ns=3, nr=20)
    k = rng.standard_normal((1, T, d)).astype(np.float32)
    v = rng.standard_normal((1, T, d)).astype(np.float32)
    oc.append(k[:, :150], v[:, :150])
    oc.append(k[:, 150:], v[:, 150:])
    q = rng.standard_normal((1, G, d)).astype(np.float32)
    out, _, lg = oc.decode(q, 0.125, want_logits=True)
    kh, vh = oc.dequant(0)
    ref, _, _, _, _ = _decode_ref(oc, d, T)
    quant = np.r_[3:T - 20]
    np.testing.assert_allclose(vh[quant], ref[quant], atol=1e-9)
    np.testing.assert_array_equal(vh[:3], fr.bf16(oc.sink_v[0, :3]))
    p = np.exp(lg[0] - lg[0].max(1, keepdims=True))
    np.testing.assert_allclose(out[0], (p / p.sum(1, keepdims=True)) @ vh, atol=1e-12)
