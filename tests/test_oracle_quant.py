"""Pins of the oracle's encoder (quantize + pack).

Asymmetric INT-b keys with channel 0 in BF16 outside the range estimate: Dual-QK: Sharp
Queries and Flat Keys for Prunable 2-bit KV Caches, sec. 3.3 and sec. C.3.  Lloyd-Max
codes after a Walsh-Hadamard rotation: TurboQuant on Quantized Models (topic list);
Statistical Inference ... Inspired by TurboQuant (scheme KQV, Beta -> Gaussian marginal).
Sink tokens in BF16: TurboQuant on Quantized Models (abstract).  Per-token INT2 values with
a clipping ratio: Dual-QK sec. 3.3 and sec. B.2.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import format_ref as fr


def _cache(oracle_mod, d=128, cap=256, kfmt=0, rot=0, ch0=0, n_sink=0, units=1, vfmt=0, vclip=1.0):
    g = oracle_mod.Geometry(batch=units, n_kv_heads=1, head_dim=d, capacity=cap, n_sink=n_sink,
                            k_format=kfmt, k_hadamard=rot, k_ch0_bf16=ch0, v_format=vfmt, v_clip=vclip)
    return oracle_mod.OracleCache(g)


def _groups(rng, n, kind):
    if kind == "normal":
        return rng.standard_normal((n, 32)).astype(np.float32)
    if kind == "t3":
        return rng.standard_t(3, (n, 32)).astype(np.float32)
    if kind == "wide":
        return (rng.standard_normal((n, 32)) * 1000).astype(np.float32)
    return (rng.uniform(-1e-3, 1e-3, (n, 32))).astype(np.float32)


@pytest.mark.parametrize("kfmt,bits", [(0, 2), (1, 4), (3, 8)])
@pytest.mark.parametrize("kind", ["normal", "t3", "wide", "tiny"])
def test_asym_codes_are_nearest_level(oracle_mod, kfmt, bits, kind):
    """Brute force: every code is the nearest of the 2^b levels zf + k*sf (fp64), except
    within 1e-4 of a midpoint where fp32 rounding may legitimately pick either side."""
    rng = np.random.default_rng(100 + bits)
    T, d = 200, 128
    x = _groups(rng, T * 4, kind).reshape(1, T, d)
    oc = _cache(oracle_mod, d=d, kfmt=kfmt)
    oc.append(x, x)
    codes = fr.key_codes(oc.k_codes[0], bits, d, T)
    s, z = fr.scale_zero(oc.k_sz[0], d, T)
    S, Z = np.repeat(s, 32, 1), np.repeat(z, 32, 1)
    qmax = (1 << bits) - 1
    levels = Z[..., None] + np.arange(qmax + 1)[None, None, :] * S[..., None]
    brute = np.argmin(np.abs(x[0].astype(np.float64)[..., None] - levels), axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (x[0] - Z) / S
    frac = np.abs(u - np.floor(u) - 0.5)
    ok = (frac > 1e-4) | ~np.isfinite(u)
    assert np.all(codes[ok] == brute[ok])
    assert codes.min() >= 0 and codes.max() <= qmax
    # parameters describe the group range: zero ~ min, zero + qmax*scale ~ max (fp16 precision)
    g = x[0].reshape(T, 4, 32).astype(np.float64)
    mn, mx = g.min(-1), g.max(-1)
    tol = 2 ** -10 * np.maximum(np.abs(mn), np.abs(mx)) + 6e-8 * qmax
    assert np.all(np.abs(z - mn) <= tol)
    assert np.all(np.abs(z + qmax * s - mx) <= 2 * tol + qmax * 2 ** -10 * s)
    # reconstruction error bound inside the range
    xh = codes * S + Z
    # fp16 rounding of the scale: half an ulp, 2^-11 relative or 2^-25 absolute (subnormal)
    s_err = np.maximum(2 ** -11 * S, 2 ** -25)
    bound = S / 2 + np.abs(Z - np.repeat(mn, 32, 1)) + qmax * s_err + 1e-6 * np.abs(x[0])
    assert np.all(np.abs(xh - x[0]) <= bound + 1e-12)


def test_channel0_protection_narrows_range(oracle_mod):
    """Dual-QK sec. C.3: keeping channel 0 out of the range estimate narrows the INT2 range
    when channel 0 sets the extremum; channel 0 is stored in BF16 and its code slot is 0."""
    rng = np.random.default_rng(5)
    T, d = 64, 128
    x = rng.standard_normal((1, T, d)).astype(np.float32)
    x[0, :, 0] = 40.0 * np.sign(rng.standard_normal(T)).astype(np.float32)
    prot = _cache(oracle_mod, ch0=1)
    plain = _cache(oracle_mod, ch0=0)
    prot.append(x, x)
    plain.append(x, x)
    sp, _ = fr.scale_zero(prot.k_sz[0], d, T)
    sn, _ = fr.scale_zero(plain.k_sz[0], d, T)
    assert np.all(sp[:, 0] < sn[:, 0])
    np.testing.assert_array_equal(sp[:, 1:], sn[:, 1:])
    assert np.all(fr.key_codes(prot.k_codes[0], 2, d, T)[:, 0] == 0)
    np.testing.assert_array_equal(fr.bf16(prot.k_ch0[0, :T]), x[0, :, 0])
    kh_p, _ = fr.decode_unit(prot, 0, T)
    kh_n, _ = fr.decode_unit(plain, 0, T)
    err_p = np.abs(kh_p[:, 1:32] - x[0, :, 1:32]).mean()
    err_n = np.abs(kh_n[:, 1:32] - x[0, :, 1:32]).mean()
    assert err_p < 0.5 * err_n


def test_degenerate_group_codes_zero(oracle_mod):
    d, T = 64, 4
    x = np.full((1, T, d), 1.2345, dtype=np.float32)
    oc = _cache(oracle_mod, d=d, kfmt=0)
    oc.append(x, x)
    assert np.all(fr.key_codes(oc.k_codes[0], 2, d, T) == 0)
    assert np.all(fr.value_codes(oc.v_codes[0], d, T) == 0)
    s, z = fr.scale_zero(oc.k_sz[0], d, T)
    assert np.all(s == 0) and np.all(z == np.float16(1.2345))
    kh, vh = fr.decode_unit(oc, 0, T)
    assert np.all(kh == np.float64(np.float16(1.2345))) and np.all(vh == kh)


def test_layout_roundtrip_two_independent_decoders(oracle_mod):
    """The oracle's C decoder and the numpy spec reader agree exactly on every format."""
    rng = np.random.default_rng(9)
    for kfmt, rot, ch0, ns, d in [(0, 0, 1, 0, 128), (1, 0, 0, 3, 64), (2, 1, 0, 2, 128),
                                  (2, 0, 0, 0, 64), (3, 0, 1, 0, 128), (0, 0, 0, 5, 64)]:
        T = 37
        oc = _cache(oracle_mod, d=d, kfmt=kfmt, rot=rot, ch0=ch0, n_sink=ns, units=2)
        x = rng.standard_normal((2, T, d)).astype(np.float32)
        v = rng.standard_normal((2, T, d)).astype(np.float32)
        oc.append(x[:, :20], v[:, :20])
        oc.append(x[:, 20:], v[:, 20:])
        for u in range(2):
            kh, vh = oc.dequant(u)
            kr, vr = fr.decode_unit(oc, u, T)
            np.testing.assert_array_equal(kh, kr)
            np.testing.assert_array_equal(vh, vr)
            # decoded values track the inputs channel by channel (catches transposed indices)
            start = ns
            err = np.abs(vh[start:] - v[u, start:]).max()
            assert err < 0.2 * np.abs(v[u]).max()
            if kfmt != 2:
                assert np.abs(kh[start:] - x[u, start:]).max() < 0.5 * np.abs(x[u]).max()


def test_sinks_store_bf16_and_skip_quantized_slots(oracle_mod):
    rng = np.random.default_rng(3)
    d, T, ns = 64, 10, 4
    oc = _cache(oracle_mod, d=d, n_sink=ns)
    x = rng.standard_normal((1, T, d)).astype(np.float32)
    v = rng.standard_normal((1, T, d)).astype(np.float32)
    oc.append(x, v)
    def torch_bf16_bits(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    np.testing.assert_array_equal(oc.sink_k[0, :ns], torch_bf16_bits(x[0, :ns]))
    np.testing.assert_array_equal(oc.sink_v[0, :ns], torch_bf16_bits(v[0, :ns]))
    np.testing.assert_array_equal(oc.k_codes[0, :, :ns], 0)
    np.testing.assert_array_equal(oc.k_sz[0, :, :ns], 0)
    np.testing.assert_array_equal(oc.v_sz[0, :, :ns], 0)
    assert np.all(oc.k_sz[0, :, ns:T] != 0)


def test_lloyd4_codes_are_nearest_centroid_and_norm(oracle_mod):
    rng = np.random.default_rng(21)
    d, T = 128, 300
    for rot in (0, 1):
        oc = _cache(oracle_mod, d=d, cap=512, kfmt=2, rot=rot)
        x = (rng.standard_normal((1, T, d)) * rng.uniform(0.1, 10, (1, T, 1))).astype(np.float32)
        oc.append(x, x)
        codes = fr.key_codes(oc.k_codes[0], 4, d, T)
        rho = fr.f16(oc.k_norm[0, :T])
        y = np.array([oracle_mod.fwht_f32(r) for r in x[0]]) if rot else x[0]
        rms = np.sqrt((y.astype(np.float64) ** 2).mean(1))
        np.testing.assert_allclose(rho, rms, rtol=2 ** -10)
        if rot:  # Parseval: rho = ||k||
            np.testing.assert_allclose(rho, np.linalg.norm(x[0].astype(np.float64), axis=1), rtol=2 ** -10)
        z = y / rho[:, None]
        cent = oc.cent.astype(np.float64)
        brute = np.argmin(np.abs(z[..., None] - cent[None, None, :]), axis=-1)
        mids = 0.5 * (cent[:-1] + cent[1:])
        near = np.min(np.abs(z[..., None] - mids[None, None, :]), axis=-1) < 1e-5
        assert np.all(codes[~near] == brute[~near])


def test_rotated_normalised_coordinates_are_gaussian(oracle_mod):
    """Statistical Inference ... Inspired by TurboQuant, "Theoretischer Rahmen": coordinates
    of a rotated unit vector are Beta((d-1)/2,(d-1)/2) and tend to a Gaussian; with the
    RMS normalisation z = y/rho the first stored coordinate is close to N(0,1) at d = 128."""
    rng = np.random.default_rng(33)
    d, T = 128, 3000
    x = (rng.standard_normal((T, d)) * np.linspace(0.2, 3.0, d)).astype(np.float32)
    y = oracle_mod.fwht_f32(x)
    rho = np.sqrt((y.astype(np.float64) ** 2).mean(1))
    z = y[:, 5] / rho
    assert stats.kstest(z, "norm").pvalue > 1e-3
    # without the rotation the same normalisation is far from Gaussian (unequal channel scales)
    rho0 = np.sqrt((x.astype(np.float64) ** 2).mean(1))
    assert stats.kstest(x[:, 5] / rho0, "norm").pvalue < 1e-6


def test_zero_key_vector(oracle_mod):
    d = 64
    oc = _cache(oracle_mod, d=d, kfmt=2, rot=1)
    x = np.zeros((1, 2, d), dtype=np.float32)
    oc.append(x, x)
    kh, vh = oc.dequant(0)
    assert np.all(kh == 0) and np.all(vh == 0)
    assert np.all(oc.k_norm[0, :2] == 0)


def test_input_validation(oracle_mod):
    oc = _cache(oracle_mod, d=64, cap=256)
    with pytest.raises(ValueError):
        oc.append(np.full((1, 1, 64), 7e4, np.float32), np.zeros((1, 1, 64), np.float32))
    with pytest.raises(ValueError):
        oc.append(np.zeros((1, 257, 64), np.float32), np.zeros((1, 257, 64), np.float32))


def _token_int2(oc, d, T):
    codes = fr.value_codes_int2(oc.v_codes[0], d, T)
    sz = oc.v_sz[0, 0, :T]
    return codes, fr.f16(sz & 0xFFFF), fr.f16(sz >> 16)


@pytest.mark.parametrize("clip", [1.0, 0.92, 0.5])
@pytest.mark.parametrize("kind", ["normal", "t3", "wide"])
def test_token_int2_codes_are_nearest_level(oracle_mod, clip, kind):
    """Per-token INT2 values with clipping (Dual-QK sec. B.2): brute force over the 4 levels
    zf + k*sf (entries beyond the clipped range land on an end level), except within 1e-4
    of a midpoint; the parameters describe the clipped range [clip*min, clip*max]."""
    rng = np.random.default_rng(300)
    T, d = 150, 128
    x = _groups(rng, T * 4, kind).reshape(1, T, d)
    oc = _cache(oracle_mod, d=d, vfmt=1, vclip=clip)
    oc.append(x, x)
    codes, s, z = _token_int2(oc, d, T)
    levels = z[:, None, None] + np.arange(4)[None, None, :] * s[:, None, None]
    brute = np.argmin(np.abs(x[0].astype(np.float64)[..., None] - levels), axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (x[0] - z[:, None]) / s[:, None]
    frac = np.abs(u - np.floor(u) - 0.5)
    ok = (frac > 1e-4) | ~np.isfinite(u)
    assert np.all(codes[ok] == brute[ok])
    mn, mx = x[0].astype(np.float64).min(-1), x[0].astype(np.float64).max(-1)
    tol = 2 ** -10 * np.maximum(np.abs(mn), np.abs(mx))
    assert np.all(np.abs(z - clip * mn) <= tol)
    assert np.all(np.abs(z + 3 * s - clip * mx) <= 3 * tol)
    # the extremes saturate at the end codes
    assert np.all(codes[np.arange(T), np.argmax(x[0], -1)] == 3)
    assert np.all(codes[np.arange(T), np.argmin(x[0], -1)] == 0)


def test_token_int2_without_clipping_is_one_group_asym2(oracle_mod):
    """With clip = 1 a per-token INT2 value is the (brute-force pinned) asymmetric INT2
    quantizer over a group spanning the whole token: same codes and parameters as INT2
    keys of a head whose 32-channel groups all hold copies of that token's extremes."""
    rng = np.random.default_rng(301)
    T, d = 64, 128
    x = rng.standard_normal((1, T, d)).astype(np.float32)
    # put each token's min and max into every 32-channel group, so every key group's
    # range equals the whole token's range
    mn, mx = x[0].min(-1), x[0].max(-1)
    for g in range(4):
        x[0, :, 32 * g] = mn
        x[0, :, 32 * g + 1] = mx
    oc = _cache(oracle_mod, d=d, vfmt=1, vclip=1.0)
    oc.append(x, x)
    codes, s, z = _token_int2(oc, d, T)
    kcodes = fr.key_codes(oc.k_codes[0], 2, d, T)
    ks, kz = fr.scale_zero(oc.k_sz[0], d, T)
    np.testing.assert_array_equal(codes, kcodes)
    for g in range(4):
        np.testing.assert_array_equal(s, ks[:, g])
        np.testing.assert_array_equal(z, kz[:, g])


def test_token_int2_clipping_lowers_gaussian_error(oracle_mod):
    """At 2 bits the uniform quantizer with least squared error on N(0,1) spans far less
    than the extremes of 128 draws, so shrinking the range by 0.92 lowers the mean squared
    error (the reason for the clipping ratio, Dual-QK sec. B.2)."""
    rng = np.random.default_rng(302)
    T, d = 400, 128
    x = rng.standard_normal((1, T, d)).astype(np.float32)
    err = {}
    for clip in (1.0, 0.92):
        oc = _cache(oracle_mod, d=d, cap=512, vfmt=1, vclip=clip)
        oc.append(x, x)
        _, vh = oc.dequant(0)
        err[clip] = np.mean((vh - x[0]) ** 2)
    assert err[0.92] < 0.97 * err[1.0]


def test_token_int2_layout_two_independent_decoders(oracle_mod):
    """C decoder and the numpy reader agree on per-token INT2 values, odd lengths and
    appends split across a token pair included; sinks stay BF16."""
    rng = np.random.default_rng(303)
    for d, ns in [(128, 0), (64, 3), (128, 5)]:
        T = 41
        oc = _cache(oracle_mod, d=d, n_sink=ns, units=2, vfmt=1, vclip=0.92)
        x = rng.standard_normal((2, T, d)).astype(np.float32)
        v = rng.standard_normal((2, T, d)).astype(np.float32)
        oc.append(x[:, :17], v[:, :17])
        oc.append(x[:, 17:], v[:, 17:])
        for u in range(2):
            kh, vh = oc.dequant(u)
            kr, vr = fr.decode_unit(oc, u, T)
            np.testing.assert_array_equal(kh, kr)
            np.testing.assert_array_equal(vh, vr)
            rmse = np.sqrt(np.mean((vh[ns:] - v[u, ns:]) ** 2))
            assert rmse < 0.6  # INT2 over ~[-2.4, 2.4]: step ~1.6, rms error ~0.45
            np.testing.assert_array_equal(vh[:ns], fr.bf16(oc.sink_v[u, :ns]))
