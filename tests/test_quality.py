"""Pins of the quality diagnostics (oracle/quality.py): the metrics against closed forms and
constructed cases, and the behaviour the KV-quantisation statistics page reports
(Statistical Inference and Quality Measures of KV Cache Quantisations Inspired by TurboQuant:
WHT protects scalar codes against heavy tails; finer codes approach exact attention)."""
import numpy as np
import pytest

import oracle
from oracle import quality as Q


def test_kl_closed_forms():
    a, b = 0.3, 0.6
    p, q = np.array([a, 1 - a]), np.array([b, 1 - b])
    want = a * np.log(a / b) + (1 - a) * np.log((1 - a) / (1 - b))
    assert Q.kl(p, q) == pytest.approx(want, rel=1e-12)
    r = np.random.default_rng(0).dirichlet(np.ones(50), size=20)
    s = np.random.default_rng(1).dirichlet(np.ones(50), size=20)
    assert np.all(Q.kl(r, s) > 0) and np.allclose(Q.kl(r, r), 0)
    assert Q.kl(np.array([1.0, 0.0]), np.array([0.5, 0.5])) == pytest.approx(np.log(2))


def test_topk_recall_constructed():
    p = np.arange(20, dtype=float)[None]  # top 5: 19..15
    assert Q.topk_recall(p, p)[0] == 1.0
    assert Q.topk_recall(p, -p)[0] == 0.0
    q = p.copy()
    q[0, [19, 18]] = -1  # two of the top five drop out
    assert Q.topk_recall(p, q)[0] == pytest.approx(3 / 5)


def test_snr_and_direction_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 64))
    assert Q.snr_db(x, x * 1.01) == pytest.approx(40.0, abs=1e-9)
    th = 0.3
    y = np.zeros((1, 64))
    y[0, 0], y[0, 1] = np.cos(th), np.sin(th)
    e = np.zeros((1, 64))
    e[0, 0] = 2.0
    assert Q.dir_err(e, y) == pytest.approx(1 - np.cos(th), abs=1e-15)


def test_eight_bit_keys_approach_exact_attention():
    m = Q.measure("gaussian", k_format=oracle.K_ASYM8, T=512)
    assert m["kl_max"] < 1e-4 and m["top5_recall"] == 1.0 and m["k_snr_db"] > 40


def test_hadamard_protects_scalar_codes_against_heavy_tails():
    """Lloyd-Max keys on Student-t(1.5) draws: with the WHT the key direction error stays at
    its Gaussian level; without it (scheme KV) it is an order of magnitude worse."""
    g = Q.measure("gaussian", k_format=oracle.K_LLOYD4, k_hadamard=1, T=1024)["k_dir"]
    w = Q.measure("t", k_format=oracle.K_LLOYD4, k_hadamard=1, T=1024, nu=1.5)["k_dir"]
    n = Q.measure("t", k_format=oracle.K_LLOYD4, k_hadamard=0, T=1024, nu=1.5)["k_dir"]
    assert w < 1.5 * g and n > 10 * w


@pytest.mark.parametrize("kind", Q.KINDS)
def test_metrics_are_finite_and_ordered(kind):
    m = Q.measure(kind, k_format=oracle.K_LLOYD4, k_hadamard=1, v_format=oracle.V_KQV, T=512)
    assert all(np.isfinite(v) for v in m.values())
    assert 0 <= m["kl_mean"] <= m["kl_max"] and 0 <= m["top5_recall"] <= 1
