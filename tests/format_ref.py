"""Independent numpy reader of the packed cache format, written from the format spec.

Used only to pin the oracle: it decodes the oracle's packed buffers a second way (numpy
bit arithmetic over whole arrays, no code shared with the oracle's C decoder), so a
wrong bit position, row, pair or group index in either one shows up as a mismatch.

Format (per unit, absolute token positions):
  keys, b-bit asymmetric or 4-bit codebook: row r of token t is word k_codes[r, t]; it holds
  channels r*(32/b) + j, j = 0..32/b-1, channel j in bits [b*j, b*j + b - 1];
  k_sz[g, t]: fp16 scale in bits 0-15, fp16 zero in bits 16-31, group g = channels 32g..32g+31;
  values: word j of token pair P = v_codes[P, j] holds channels 4j..4j+3, token 2P in the
  low 16 bits and token 2P+1 in the high 16 bits, channel 4j+k at nibble k of its half;
  v_sz like k_sz.
  Per-token INT2 values (value format 1): word j of token pair P = v_codes[P, j] holds
  channels 8j..8j+7, token 2P in the low 16 bits and 2P+1 in the high 16 bits, channel
  8j+k at bits [2k, 2k+1] of its half; v_sz[0, t] holds the token's fp16 scale and zero.
  Recent window of W positions: positions t >= max(n_sink, len - W) are read as BF16 from
  ring slot t mod W of recent_k / recent_v (keys in stored coordinates).
"""
import numpy as np


def f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def key_codes(k_codes_unit, bits, d, len_):
    """[len, d] integer codes from k_codes[R, cap]."""
    per = 32 // bits
    R = d // per
    w = k_codes_unit[:R, :len_].astype(np.uint64)  # [R, T]
    shifts = (np.arange(per, dtype=np.uint64) * bits)[None, :, None]
    codes = (w[:, None, :] >> shifts) & np.uint64((1 << bits) - 1)  # [R, per, T]
    return codes.reshape(R * per, len_).T.astype(np.int64)


def value_codes(v_codes_unit, d, len_):
    """[len, d] integer codes from v_codes[cap/2, d/4]."""
    npair = (len_ + 1) // 2
    w = v_codes_unit[:npair].astype(np.uint64)  # [P, d/4]
    halves = np.stack([w & np.uint64(0xFFFF), w >> np.uint64(16)], axis=1)  # [P, 2, d/4]
    nib = np.stack([(halves >> np.uint64(4 * k)) & np.uint64(0xF) for k in range(4)], axis=-1)
    return nib.reshape(npair * 2, d)[:len_].astype(np.int64)


def value_codes_int2(v_codes_unit, d, len_):
    """[len, d] integer codes from per-token INT2 v_codes[cap/2, d/8]."""
    npair = (len_ + 1) // 2
    w = v_codes_unit[:npair, : d // 8].astype(np.uint64)  # [P, d/8]
    halves = np.stack([w & np.uint64(0xFFFF), w >> np.uint64(16)], axis=1)  # [P, 2, d/8]
    crumbs = np.stack([(halves >> np.uint64(2 * k)) & np.uint64(3) for k in range(8)], axis=-1)
    return crumbs.reshape(npair * 2, d)[:len_].astype(np.int64)


def scale_zero(sz_unit, d, len_):
    """(scale, zero) fp64 [len, d/32] from sz[d/32, cap]."""
    s = sz_unit[: d // 32, :len_]
    return f16(s & 0xFFFF).T, f16(s >> 16).T


def decode_unit(oc, u, len_):
    """Decoded keys (stored coordinates) and values, fp64 [len, d], for unit u of an
    oracle.OracleCache (any key format)."""
    g = oc.geo
    d, ns = g.head_dim, g.n_sink
    kh = np.zeros((len_, d))
    vh = np.zeros((len_, d))
    if g.k_format == 2:  # Lloyd-Max
        codes = key_codes(oc.k_codes[u], 4, d, len_)
        rho = f16(oc.k_norm[u, :len_])
        kh[:] = rho[:, None] * oc.cent.astype(np.float64)[codes]
    else:
        codes = key_codes(oc.k_codes[u], g.key_bits, d, len_)
        s, z = scale_zero(oc.k_sz[u], d, len_)
        kh[:] = codes * np.repeat(s, 32, axis=1) + np.repeat(z, 32, axis=1)
        if g.k_ch0_bf16:
            kh[:, 0] = bf16(oc.k_ch0[u, :len_])
    if getattr(g, "v_format", 0) == 1:
        vc = value_codes_int2(oc.v_codes[u], d, len_)
        sz = oc.v_sz[u, 0, :len_]
        vh[:] = vc * f16(sz & 0xFFFF)[:, None] + f16(sz >> 16)[:, None]
    else:
        vc = value_codes(oc.v_codes[u], d, len_)
        s, z = scale_zero(oc.v_sz[u], d, len_)
        vh[:] = vc * np.repeat(s, 32, axis=1) + np.repeat(z, 32, axis=1)
    n = min(ns, len_)
    if n:
        kh[:n] = bf16(oc.sink_k[u, :n])
        vh[:n] = bf16(oc.sink_v[u, :n])
    W = getattr(g, "n_recent", 0)
    if W:
        for t in range(max(ns, len_ - W), len_):
            kh[t] = bf16(oc.recent_k[u, t % W])
            vh[t] = bf16(oc.recent_v[u, t % W])
    return kh, vh
