"""Pins of the oracle's attention over the decoded cache.

The oracle's attention is the plain definition softmax(sm * q.k^) weighted over v^ with
one softmax over all positions (Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit
KV Caches, sec. 3.4).  It is pinned here against a numpy brute force built on the
independent format reader, against closed forms, against the softmax shift invariance
(the row-mean component that softmax ignores: CASK-Q, Method), against the divergence bound
KL(p||q) <= 1/4 ||dc||^2 for a centred logit error dc (CASK-Q, Method), and against the
convergence of 8-bit codes to dense attention.
"""
import numpy as np
import pytest

import format_ref as fr


def _geo(oracle_mod, d, cap=512, kfmt=0, rot=0, ch0=0, ns=0, units=1, vfmt=0, vclip=1.0, nr=0):
    return oracle_mod.Geometry(batch=units, n_kv_heads=1, head_dim=d, capacity=cap, n_sink=ns,
                               k_format=kfmt, k_hadamard=rot, k_ch0_bf16=ch0, v_format=vfmt, v_clip=vclip,
                               n_recent=nr)


def _brute(oracle_mod, oc, q, sm, keep):
    """numpy fp64 attention from the independently decoded cache; the mask comes from the
    separately pinned ranking."""
    U, G, d = q.shape
    out = np.zeros((U, G, d))
    for u in range(U):
        kh, vh = fr.decode_unit(oc, u, oc.len)
        qs = q[u].astype(np.float64)
        rot = oc.geo.k_hadamard
        if rot:
            import scipy.linalg
            H = scipy.linalg.hadamard(d).astype(np.float64)
            qs = qs @ H.T
        qt32 = oracle_mod.fwht_f32(q[u]) if rot else q[u]
        m = oracle_mod.prune_mask(qt32, keep)
        cmask = np.array([(m >> (c // 16)) & 1 for c in range(d)], dtype=bool)
        lg = sm * (qs[:, cmask] @ kh[:, cmask].T) / (d if rot else 1)
        lg -= lg.max(1, keepdims=True)
        p = np.exp(lg)
        p /= p.sum(1, keepdims=True)
        out[u] = p @ vh
    return out


CASES = [
    # d, kfmt, rot, ch0, n_sink, T, G, keep, value format
    (64, 0, 0, 1, 0, 1, 1, 0, 0),
    (64, 0, 0, 1, 0, 7, 1, 0, 0),
    (128, 0, 0, 1, 0, 8, 4, 5, 0),
    (128, 1, 0, 0, 2, 6, 4, 0, 0),
    (128, 2, 1, 0, 0, 5, 4, 3, 0),
    (64, 2, 0, 0, 3, 8, 2, 0, 0),
    (128, 0, 0, 0, 4, 8, 8, 7, 0),
    (64, 3, 0, 1, 0, 4, 1, 2, 0),
    (128, 0, 0, 1, 3, 9, 4, 5, 1),
    (64, 1, 0, 0, 0, 7, 2, 0, 1),
]
# recent BF16 window cases: (d, kfmt, rot, ch0, n_sink, T, G, keep, value format, window)
WCASES = [(128, 0, 0, 1, 2, 9, 4, 5, 0, 3), (64, 2, 1, 0, 0, 8, 2, 0, 1, 1), (128, 1, 0, 0, 1, 6, 4, 0, 0, 16)]


@pytest.mark.parametrize("d,kfmt,rot,ch0,ns,T,G,keep,vfmt,nr", [c + (0,) for c in CASES] + WCASES)
def test_oracle_equals_bruteforce(oracle_mod, d, kfmt, rot, ch0, ns, T, G, keep, vfmt, nr):
    rng = np.random.default_rng(d + 10 * kfmt + T)
    U = 2
    oc = oracle_mod.OracleCache(_geo(oracle_mod, d, kfmt=kfmt, rot=rot, ch0=ch0, ns=ns, units=U,
                                     vfmt=vfmt, vclip=0.92, nr=nr))
    k = (rng.standard_normal((U, T, d)) * 2).astype(np.float32)
    v = rng.standard_normal((U, T, d)).astype(np.float32)
    oc.append(k, v)
    q = rng.standard_normal((U, G, d)).astype(np.float32)
    sm = 1.0 / np.sqrt(d)
    out, _ = oc.decode(q, sm, keep)
    np.testing.assert_allclose(out, _brute(oracle_mod, oc, q, sm, keep), rtol=1e-12, atol=1e-12)


def test_closed_forms(oracle_mod):
    rng = np.random.default_rng(1)
    d = 64
    # T = 1: output is the single decoded value
    oc = oracle_mod.OracleCache(_geo(oracle_mod, d, ch0=1))
    k = rng.standard_normal((1, 1, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, d)).astype(np.float32)
    oc.append(k, v)
    out, _ = oc.decode(rng.standard_normal((1, 3, d)).astype(np.float32), 0.125)
    _, vh = oc.dequant(0)
    for h in range(3):
        np.testing.assert_allclose(out[0, h], vh[0], rtol=0, atol=1e-15)
    # q = 0: uniform weights, output is the mean decoded value
    oc = oracle_mod.OracleCache(_geo(oracle_mod, d, kfmt=1, ns=2))
    k = rng.standard_normal((1, 50, d)).astype(np.float32)
    v = rng.standard_normal((1, 50, d)).astype(np.float32)
    oc.append(k, v)
    out, _ = oc.decode(np.zeros((1, 2, d), np.float32), 0.125)
    _, vh = oc.dequant(0)
    np.testing.assert_allclose(out[0, 0], vh.mean(0), rtol=1e-13, atol=1e-14)
    # identical keys: uniform weights whatever the query
    oc = oracle_mod.OracleCache(_geo(oracle_mod, d, kfmt=2, rot=1))
    k = np.repeat(rng.standard_normal((1, 1, d)).astype(np.float32), 40, axis=1)
    v = rng.standard_normal((1, 40, d)).astype(np.float32)
    oc.append(k, v)
    out, _ = oc.decode(rng.standard_normal((1, 4, d)).astype(np.float32) * 5, 0.125)
    _, vh = oc.dequant(0)
    np.testing.assert_allclose(out[0, 3], vh.mean(0), rtol=1e-12, atol=1e-13)


def test_softmax_shift_invariance(oracle_mod):
    """Adding the same constant to every key zero point shifts every logit of a head by
    the same amount (sm * delta * sum of kept non-protected q channels); outputs unchanged."""
    rng = np.random.default_rng(2)
    d, T, G = 128, 200, 4
    oc = oracle_mod.OracleCache(_geo(oracle_mod, d, ch0=1))
    oc.append(rng.standard_normal((1, T, d)).astype(np.float32),
              rng.standard_normal((1, T, d)).astype(np.float32))
    q = rng.standard_normal((1, G, d)).astype(np.float32)
    base, _, lg0 = oc.decode(q, 0.088, 6, want_logits=True)
    z = (oc.k_sz[0, :, :T] >> 16).astype(np.uint16).view(np.float16)
    z2 = (z.astype(np.float64) + 0.5).astype(np.float16)  # exact in fp16 for |z| < 512
    assert np.all(z2.astype(np.float64) == z.astype(np.float64) + 0.5)
    oc.k_sz[0, :, :T] = (oc.k_sz[0, :, :T] & 0xFFFF) | (z2.view(np.uint16).astype(np.uint32) << 16)
    shifted, _, lg1 = oc.decode(q, 0.088, 6, want_logits=True)
    diff = lg1 - lg0
    assert np.ptp(diff, axis=-1).max() < 1e-12 and np.abs(diff).max() > 1e-3
    np.testing.assert_allclose(shifted, base, rtol=1e-12, atol=1e-12)


def test_eight_bit_codes_converge_to_dense(oracle_mod):
    rng = np.random.default_rng(3)
    d, T, G = 64, 128, 4
    k = rng.standard_normal((1, T, d)).astype(np.float32)
    v = rng.standard_normal((1, T, d)).astype(np.float32)
    q = rng.standard_normal((1, G, d)).astype(np.float32)
    sm = 0.125
    lg = sm * q[0].astype(np.float64) @ k[0].astype(np.float64).T
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    dense = p @ v[0].astype(np.float64)
    errs = []
    for kfmt in (0, 1, 3):  # 2, 4, 8 bits on keys (values stay INT4)
        oc = oracle_mod.OracleCache(_geo(oracle_mod, d, kfmt=kfmt))
        oc.append(k, v)
        out, _ = oc.decode(q, sm)
        kh, _ = oc.dequant(0)
        lgq = sm * q[0].astype(np.float64) @ kh.T
        pq = np.exp(lgq - lgq.max(1, keepdims=True))
        pq /= pq.sum(1, keepdims=True)
        errs.append(np.abs(pq - p).sum(1).max())
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 1e-2
    # with 8-bit keys the whole output is within the INT4 value error of dense attention
    oc = oracle_mod.OracleCache(_geo(oracle_mod, d, kfmt=3))
    oc.append(k, v)
    out, _ = oc.decode(q, sm)
    rel = np.linalg.norm(out[0] - dense, axis=1) / np.linalg.norm(dense, axis=1)
    assert rel.max() < 0.1


@pytest.mark.parametrize("kfmt,rot", [(0, 0), (2, 1), (1, 0)])
def test_kl_bound_on_centred_logit_error(oracle_mod, kfmt, rot):
    """CASK-Q, Method: KL(p||q) <= 1/4 ||dc||^2 where dc is the row-centred logit error."""
    rng = np.random.default_rng(4)
    d, T, G = 128, 256, 4
    k = rng.standard_normal((1, T, d)).astype(np.float32)
    oc = oracle_mod.OracleCache(_geo(oracle_mod, d, kfmt=kfmt, rot=rot))
    oc.append(k, rng.standard_normal((1, T, d)).astype(np.float32))
    q = rng.standard_normal((1, G, d)).astype(np.float32)
    sm = 1 / np.sqrt(d)
    _, _, lq = oc.decode(q, sm, want_logits=True)
    ld = sm * q[0].astype(np.float64) @ k[0].astype(np.float64).T
    for h in range(G):
        a, b = ld[h], lq[0, h]
        p = np.exp(a - a.max()); p /= p.sum()
        qq = np.exp(b - b.max()); qq /= qq.sum()
        kl = float(np.sum(p * (np.log(p) - np.log(qq))))
        dc = (b - a) - (b - a).mean()
        assert 0 <= kl <= 0.25 * float(dc @ dc)
