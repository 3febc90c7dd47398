"""Pins of the oracle's recent BF16 window.

Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV Caches, sec. 3.3 and 4.1: the most
recent 256 positions stay in BF16 beside the first 64.  TurboQuant on Quantized Models
(abstract): past-only quantization -- the newest tokens attend unquantized.  Reading: a
position enters ring slot t mod W in BF16 (keys in stored coordinates) and is quantised from
that BF16 copy when position t + W takes the slot.
"""
import numpy as np
import pytest
import torch

import format_ref as fr


def _cache(oracle_mod, d=128, cap=512, kfmt=0, rot=0, ch0=0, ns=0, nr=0, units=1, vfmt=0):
    g = oracle_mod.Geometry(batch=units, n_kv_heads=1, head_dim=d, capacity=cap, n_sink=ns, k_format=kfmt,
                            k_hadamard=rot, k_ch0_bf16=ch0, v_format=vfmt, v_clip=0.92, n_recent=nr)
    return oracle_mod.OracleCache(g)


def _bf16(x):
    """bf16 rounding by torch (round to nearest even), back to fp64."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("rot,ns,T,W", [(0, 0, 40, 64), (1, 3, 50, 47), (0, 5, 5, 8), (1, 0, 1, 1)])
def test_window_covering_all_positions_is_dense_bf16_attention(oracle_mod, rot, ns, T, W):
    """When every position is a sink or in the window, attention is the plain softmax over
    the BF16-rounded keys (stored coordinates) and values: numpy closed form."""
    import scipy.linalg
    rng = np.random.default_rng(400 + T)
    d, G = 128, 4
    oc = _cache(oracle_mod, d=d, kfmt=2 if rot else 0, rot=rot, ns=ns, nr=W)
    k = rng.standard_normal((1, T, d)).astype(np.float32)
    v = rng.standard_normal((1, T, d)).astype(np.float32)
    oc.append(k, v)
    q = rng.standard_normal((1, G, d)).astype(np.float32)
    sm = 1.0 / np.sqrt(d)
    out, _ = oc.decode(q, sm)
    ks = oracle_mod.fwht_f32(k[0]) if rot else k[0]  # stored coordinates in fp32
    kb, vb = _bf16(ks), _bf16(v[0])
    qs = q[0].astype(np.float64)
    if rot:
        qs = qs @ scipy.linalg.hadamard(d).astype(np.float64).T
    lg = sm * (qs @ kb.T) / (d if rot else 1)
    p = np.exp(lg - lg.max(1, keepdims=True))
    ref = (p / p.sum(1, keepdims=True)) @ vb
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)
    assert not oc.k_codes.any() and not oc.v_codes.any()  # nothing quantised yet


@pytest.mark.parametrize("kfmt,rot,ch0,vfmt", [(0, 0, 1, 0), (2, 1, 0, 1), (1, 0, 0, 0)])
def test_left_positions_are_quantised_from_their_bf16_copy(oracle_mod, kfmt, rot, ch0, vfmt):
    """Codes of positions that left the window equal those of a window-less cache (no
    rotation) fed the BF16-rounded stored-coordinate inputs; positions still in the window
    are not written to the quantised arrays."""
    rng = np.random.default_rng(410 + kfmt)
    d, T, W, ns = 128, 90, 24, 3
    k = (rng.standard_normal((1, T, d)) * 3).astype(np.float32)
    v = rng.standard_normal((1, T, d)).astype(np.float32)
    win = _cache(oracle_mod, kfmt=kfmt, rot=rot, ch0=ch0, ns=ns, nr=W, vfmt=vfmt)
    win.append(k[:, :31], v[:, :31])
    win.append(k[:, 31:], v[:, 31:])
    ks = oracle_mod.fwht_f32(k[0])[None] if rot else k
    plain = _cache(oracle_mod, kfmt=kfmt, rot=0, ch0=ch0, ns=ns, vfmt=vfmt)
    plain.append(_bf16(ks).astype(np.float32), _bf16(v).astype(np.float32))
    q_end = T - W
    for name in ("k_codes", "k_sz", "k_norm", "k_ch0", "v_sz"):
        a, b = getattr(win, name), getattr(plain, name)
        np.testing.assert_array_equal(a[..., :q_end], b[..., :q_end], err_msg=name)
        assert not a[..., q_end:].any(), name
    # value codes: pairs fully below q_end match, the window's are untouched
    np.testing.assert_array_equal(win.v_codes[:, : q_end // 2], plain.v_codes[:, : q_end // 2])
    assert not win.v_codes[:, (q_end + 1) // 2:].any()
    np.testing.assert_array_equal(win.sink_k, plain.sink_k)


def test_ring_holds_the_most_recent_positions(oracle_mod):
    """Slot t mod W holds the BF16 stored-coordinate key / value of each of the last W
    positions, whatever the append cut; earlier appends were overwritten."""
    rng = np.random.default_rng(420)
    d, T, W, ns = 64, 77, 10, 4
    k = rng.standard_normal((1, T, d)).astype(np.float32)
    v = rng.standard_normal((1, T, d)).astype(np.float32)
    for cuts in ([T], [1] * T, [30, 1, 46], [7, 70]):
        oc = _cache(oracle_mod, d=d, kfmt=1, ns=ns, nr=W)
        t = 0
        for n in cuts:
            oc.append(k[:, t:t + n], v[:, t:t + n])
            t += n
        for pos in range(T - W, T):
            np.testing.assert_array_equal(fr.bf16(oc.recent_k[0, pos % W]), _bf16(k[0, pos]))
            np.testing.assert_array_equal(fr.bf16(oc.recent_v[0, pos % W]), _bf16(v[0, pos]))
        if cuts == [T]:
            first = oc
        else:
            for name in ("k_codes", "k_sz", "v_codes", "v_sz", "sink_k", "sink_v", "recent_k", "recent_v"):
                np.testing.assert_array_equal(getattr(oc, name), getattr(first, name), err_msg=name)


def test_window_of_one_is_past_only(oracle_mod):
    """W = 1: the newest position attends in BF16, all earlier ones quantised -- the brute
    force over the independently decoded cache, with the newest key and value replaced by
    their BF16 roundings, gives the same output."""
    rng = np.random.default_rng(430)
    d, T, G = 128, 33, 4
    k = rng.standard_normal((1, T, d)).astype(np.float32)
    v = rng.standard_normal((1, T, d)).astype(np.float32)
    oc = _cache(oracle_mod, nr=1)
    oc.append(k, v)
    kh, vh = fr.decode_unit(oc, 0, T)
    np.testing.assert_array_equal(kh[-1], _bf16(k[0, -1]))
    np.testing.assert_array_equal(vh[-1], _bf16(v[0, -1]))
    plain = _cache(oracle_mod)
    plain.append(_bf16(k).astype(np.float32), _bf16(v).astype(np.float32))
    kp, vp = fr.decode_unit(plain, 0, T)
    np.testing.assert_array_equal(kh[:-1], kp[:-1])
    np.testing.assert_array_equal(vh[:-1], vp[:-1])
    q = rng.standard_normal((1, G, d)).astype(np.float32)
    sm = 1.0 / np.sqrt(d)
    out, _ = oc.decode(q, sm)
    lg = sm * (q[0].astype(np.float64) @ kh.T)
    p = np.exp(lg - lg.max(1, keepdims=True))
    np.testing.assert_allclose(out[0], (p / p.sum(1, keepdims=True)) @ vh, rtol=1e-12, atol=1e-12)
