"""Pins of the oracle's query-channel-group pruning mask.

Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV Caches, sec. 3.2 (keep the m
channel groups with the largest group-level query norms, one shared mask per step),
sec. C.2 (group-L2 keeps the most query energy for a fixed budget; energy summed over
the GQA group's heads), App. A (every key channel stays stored; the mask only selects
what is read).
"""
import itertools

import numpy as np
import pytest


@pytest.mark.parametrize("G,d", [(4, 128), (1, 64), (8, 128), (2, 64)])
def test_mask_maximises_group_energy_exhaustively(oracle_mod, G, d):
    rng = np.random.default_rng(G * 1000 + d)
    P = d // 16
    for _ in range(60):
        q = (rng.standard_normal((G, d)) * rng.uniform(0.1, 5, (1, d))).astype(np.float32)
        E = (q.astype(np.float64) ** 2).reshape(G, P, 16).sum((0, 2))
        for m in range(1, P):
            mask = oracle_mod.prune_mask(q, m)
            kept = [p for p in range(P) if mask >> p & 1]
            assert len(kept) == m
            best = max(sum(E[list(s)]) for s in itertools.combinations(range(P), m))
            assert sum(E[kept]) >= best * (1 - 1e-6)


def test_mask_no_pruning_cases(oracle_mod):
    q = np.random.default_rng(0).standard_normal((4, 128)).astype(np.float32)
    for m in (0, -3, 8, 9, 100):
        assert oracle_mod.prune_mask(q, m) == 0xFF
    q64 = q[:, :64].copy()
    assert oracle_mod.prune_mask(q64, 4) == 0xF


def test_mask_ties_go_to_lower_group(oracle_mod):
    q = np.ones((4, 128), dtype=np.float32)
    for m in range(1, 8):
        assert oracle_mod.prune_mask(q, m) == (1 << m) - 1
    q[:, 16 * 6:16 * 7] = 2.0  # group 6 strictly largest
    assert oracle_mod.prune_mask(q, 1) == 1 << 6
    assert oracle_mod.prune_mask(q, 2) == (1 << 6) | 1


def test_mask_sums_heads_of_gqa_group(oracle_mod):
    """A group that is large for one head only loses to a group moderately large for all."""
    q = np.full((4, 64), 0.1, dtype=np.float32)
    q[0, 0:16] = 3.0  # group 0: energy 16*9 = 144 on head 0 only
    q[:, 16:32] = 1.8  # group 1: 16*3.24*4 = 207 summed over heads
    assert oracle_mod.prune_mask(q, 1) == 0b10
    assert oracle_mod.prune_mask(q[:1], 1) == 0b01


def _cfg_cache(oracle_mod, kfmt=0, rot=0, ch0=1, d=128, T=300, units=3, seed=0, ns=0):
    rng = np.random.default_rng(seed)
    g = oracle_mod.Geometry(batch=units, n_kv_heads=1, head_dim=d, capacity=512, n_sink=ns,
                            k_format=kfmt, k_hadamard=rot, k_ch0_bf16=ch0)
    oc = oracle_mod.OracleCache(g)
    k = rng.standard_normal((units, T, d)).astype(np.float32)
    v = rng.standard_normal((units, T, d)).astype(np.float32)
    oc.append(k, v)
    return oc, rng


@pytest.mark.parametrize("kfmt,rot,ch0", [(0, 0, 1), (2, 1, 0), (1, 0, 0)])
def test_keep_all_equals_no_pruning_and_cache_untouched(oracle_mod, kfmt, rot, ch0):
    oc, rng = _cfg_cache(oracle_mod, kfmt, rot, ch0)
    before = [a.copy() for a in (oc.k_codes, oc.k_sz, oc.k_norm, oc.k_ch0, oc.v_codes, oc.v_sz)]
    q = rng.standard_normal((oc.U, 4, 128)).astype(np.float32)
    o0, m0 = oc.decode(q, 0.088, 0)
    o8, m8 = oc.decode(q, 0.088, 8)
    o5, m5 = oc.decode(q, 0.088, 5)
    np.testing.assert_array_equal(o0, o8)
    assert np.all(m0 == 0xFF) and np.all(m8 == 0xFF)
    assert all(bin(int(m)).count("1") == 5 for m in m5)
    assert not np.array_equal(o0, o5)
    after = (oc.k_codes, oc.k_sz, oc.k_norm, oc.k_ch0, oc.v_codes, oc.v_sz)
    for a, b in zip(before, after):
        np.testing.assert_array_equal(a, b)


def test_mask_uses_rotated_coordinates(oracle_mod):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    oc, _ = _cfg_cache(oracle_mod, kfmt=2, rot=1, ch0=0, units=1, T=10)
    _, m = oc.decode(q[None], 0.088, 3)
    assert int(m[0]) == oracle_mod.prune_mask(oracle_mod.fwht_f32(q), 3)
