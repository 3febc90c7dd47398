"""CPU oracle for low-bit KV-cache decode attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product library (``bit_kv_cache_kvq_amd``) never imports,
links or calls it, and the two share no code: the only thing both sides use is the
seeded input generator module ``bit_kv_cache_kvq_amd.synth``, which holds none of the
method's arithmetic.

The arithmetic lives in ``kvq_oracle.c`` (plain C, fp32 fixed-order encoding, fp64
decoding and attention); this module builds it with gcc and marshals numpy arrays.
See ``kvq_oracle.c`` for what each function computes and the passages it follows.
``quality.py`` builds the quality diagnostics (KL, routing recall, scale and direction
errors) on top of it.

Parity status: every function is pinned by the CPU tests (``tests/test_oracle_*.py``)
against library conversions, explicit matrices, brute force, closed forms or the
published Lloyd-Max table; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# fixed-order IEEE fp32 for the encoder: no contraction, no fast-math, SSE arithmetic
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-Wall", "-Wextra"]

K_ASYM2, K_ASYM4, K_LLOYD4, K_ASYM8 = 0, 1, 2, 3
V_ASYM4_G32, V_ASYM2_TOKEN, V_KQV = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile liboracle.so in place with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_f16_array.argtypes = [P, P, ctypes.c_size_t]
        L.oracle_f16_to_f32_array.argtypes = [P, P, ctypes.c_size_t]
        L.oracle_f32_to_bf16_array.argtypes = [P, P, ctypes.c_size_t]
        L.oracle_fwht_f32.argtypes = [P, i]
        L.oracle_fwht_f64.argtypes = [P, i]
        L.oracle_tree_sum_f32.restype = ctypes.c_float
        L.oracle_tree_sum_f32.argtypes = [P, i]
        L.oracle_lloyd_max_gaussian.restype = i
        L.oracle_lloyd_max_gaussian.argtypes = [i, ctypes.c_double, i, P, P]
        cache_args = [i, i, i, i, i, i, i, ctypes.c_float, i, P, P, P, P, P, P, P, P, P, P, i, P, P, P, P]
        L.oracle_quant_append.argtypes = cache_args + [P, P, i, i, i, P, P]
        L.oracle_prune_mask.restype = ctypes.c_uint32
        L.oracle_prune_mask.argtypes = [P, i, i, i]
        L.oracle_dequant_unit.argtypes = cache_args + [P, i, i, P, P]
        L.oracle_decode_attn.argtypes = cache_args + [P, i, i, i, P, ctypes.c_double, i, P, P, P]
        L.oracle_num_threads.restype = i
        L.oracle_set_num_threads.argtypes = [i]
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ scalar / vector ops
def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    h = np.empty(x.size, dtype=np.uint16)
    lib().oracle_f32_to_f16_array(_p(x), _p(h), x.size)
    return h


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    x = np.empty(h.size, dtype=np.float32)
    lib().oracle_f16_to_f32_array(_p(h), _p(x), h.size)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    h = np.empty(x.size, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(_p(x), _p(h), x.size)
    return h


def _rows(fn, x: np.ndarray, dtype) -> np.ndarray:
    y = np.array(x, dtype=dtype, copy=True, order="C")
    flat = y.reshape(-1, y.shape[-1])
    for r in range(flat.shape[0]):
        fn(_p(flat[r]), flat.shape[1])
    return y


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of every row (last axis), fp32."""
    return _rows(lib().oracle_fwht_f32, x, np.float32)


def fwht_f64(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of every row (last axis), fp64."""
    return _rows(lib().oracle_fwht_f64, x, np.float64)


def tree_sum_f32(x: np.ndarray) -> np.float32:
    y = np.array(x, dtype=np.float32, copy=True, order="C")
    return np.float32(lib().oracle_tree_sum_f32(_p(y), y.size))


def lloyd_max_gaussian(levels: int = 16, tol: float = 1e-13, max_iter: int = 200000):
    """fp64 symmetric Lloyd-Max codebook for N(0,1): (centroids, thresholds, iterations)."""
    c = np.zeros(levels, dtype=np.float64)
    t = np.zeros(levels - 1, dtype=np.float64)
    it = lib().oracle_lloyd_max_gaussian(levels, tol, max_iter, _p(c), _p(t))
    return c, t, it


def codebook_f32(levels: int = 16):
    """Stored codebook: fp32 centroids and fp32 midpoint thresholds (midpoints in fp64)."""
    c, t, _ = lloyd_max_gaussian(levels)
    return c.astype(np.float32), t.astype(np.float32)


def prune_mask(qt: np.ndarray, m: int) -> int:
    qt = np.ascontiguousarray(qt, dtype=np.float32)
    G, d = qt.shape
    return int(lib().oracle_prune_mask(_p(qt), G, d, m))


# ------------------------------------------------------------------ cache
@dataclass
class Geometry:
    batch: int
    n_kv_heads: int
    head_dim: int
    capacity: int
    n_sink: int = 0
    k_format: int = K_ASYM2
    k_hadamard: int = 0
    k_ch0_bf16: int = 0
    v_format: int = V_ASYM4_G32
    v_clip: float = 1.0
    n_recent: int = 0
    rope_bucket: int = 0

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def key_bits(self) -> int:
        return {K_ASYM2: 2, K_ASYM4: 4, K_LLOYD4: 4, K_ASYM8: 8}[self.k_format]

    @property
    def rope_buckets(self) -> int:
        """Buckets of the capacity under bucket-relative RoPE, else 1."""
        return -(-self.capacity // self.rope_bucket) if self.rope_bucket > 0 else 1


class OracleCache:
    """Host-side packed cache with the same byte layout the format defines."""

    def __init__(self, geo: Geometry, units: int | None = None, rope_table: np.ndarray | None = None,
                 qjl_signs: np.ndarray | None = None):
        """rope_table: bucket-relative RoPE's anchor (cos, sin) table, fp32
        [geo.rope_buckets][d/2][2] (an input, like the keys).  qjl_signs: KQV values' random
        sign diagonal of the sketch, uint32 [d/32], bit i set = channel i negated (an input,
        the random draw the method makes)."""
        self.geo = geo
        U = geo.units if units is None else units
        self.U = U
        d, cap = geo.head_dim, geo.capacity
        R = d * geo.key_bits // 32
        ns = max(geo.n_sink, 1)
        self.k_codes = np.zeros((U, R, cap), dtype=np.uint32)
        self.k_sz = np.zeros((U, d // 32, cap), dtype=np.uint32)
        self.k_norm = np.zeros((U, cap), dtype=np.uint16)
        self.k_ch0 = np.zeros((U, cap), dtype=np.uint16)
        per_token = geo.v_format in (V_ASYM2_TOKEN, V_KQV)
        int2_tok = geo.v_format == V_ASYM2_TOKEN
        self.v_codes = np.zeros((U, cap // 2, d // 8 if int2_tok else d // 4), dtype=np.uint32)
        self.v_sz = np.zeros((U, 1 if per_token else d // 32, cap), dtype=np.uint32)
        self.sink_k = np.zeros((U, ns, d), dtype=np.uint16)
        self.sink_v = np.zeros((U, ns, d), dtype=np.uint16)
        nr = max(geo.n_recent, 1)
        self.recent_k = np.zeros((U, nr, d), dtype=np.uint16)
        self.recent_v = np.zeros((U, nr, d), dtype=np.uint16)
        self.len = 0
        if geo.rope_bucket > 0:
            if rope_table is None:
                raise ValueError("bucket-relative RoPE needs its anchor table")
            self.rope_cs = np.ascontiguousarray(rope_table, dtype=np.float32).reshape(geo.rope_buckets, d // 2, 2)
        else:
            self.rope_cs = np.zeros((1, 1, 2), dtype=np.float32)
        self.vcent, self.vthr = codebook_f32(8)
        if geo.v_format == V_KQV:
            if qjl_signs is None:
                raise ValueError("KQV values need the sketch's random signs")
            self.qjl = np.ascontiguousarray(qjl_signs, dtype=np.uint32).reshape(d // 32)
        else:
            self.qjl = np.zeros(d // 32, dtype=np.uint32)
        if geo.k_format == K_LLOYD4:
            self.cent, self.thr = codebook_f32(16)
        else:
            self.cent = np.zeros(16, dtype=np.float32)
            self.thr = np.zeros(15, dtype=np.float32)

    def _cache_args(self):
        g = self.geo
        return [g.head_dim, g.capacity, g.n_sink, g.k_format, g.k_hadamard, g.k_ch0_bf16,
                g.v_format, float(g.v_clip), g.n_recent, _p(self.k_codes), _p(self.k_sz), _p(self.k_norm),
                _p(self.k_ch0), _p(self.v_codes), _p(self.v_sz), _p(self.sink_k), _p(self.sink_v),
                _p(self.recent_k), _p(self.recent_v), g.rope_bucket, _p(self.rope_cs),
                _p(self.vcent), _p(self.vthr), _p(self.qjl)]

    def append(self, k_new: np.ndarray, v_new: np.ndarray):
        """k_new, v_new: fp32 [U, n_new, d]; writes positions [len, len+n_new)."""
        k_new = np.ascontiguousarray(k_new, dtype=np.float32)
        v_new = np.ascontiguousarray(v_new, dtype=np.float32)
        U, n_new, d = k_new.shape
        assert U == self.U and d == self.geo.head_dim and v_new.shape == k_new.shape
        if self.len + n_new > self.geo.capacity:
            raise ValueError("capacity exceeded")
        if not (np.all(np.isfinite(k_new)) and np.all(np.isfinite(v_new))):
            raise ValueError("inputs must be finite")
        if max(np.abs(k_new).max(initial=0), np.abs(v_new).max(initial=0)) >= 6.0e4:
            raise ValueError("inputs must satisfy |x| < 6e4 so fp16 parameters stay finite")
        lib().oracle_quant_append(*self._cache_args(), _p(self.cent), _p(self.thr),
                                  U, self.len, n_new, _p(k_new), _p(v_new))
        self.len += n_new

    def dequant(self, unit: int):
        """Decoded (keys in stored coordinates, values), fp64 [len, d] each."""
        d = self.geo.head_dim
        kh = np.zeros((self.len, d), dtype=np.float64)
        vh = np.zeros((self.len, d), dtype=np.float64)
        lib().oracle_dequant_unit(*self._cache_args(), _p(self.cent), unit, self.len,
                                  _p(kh), _p(vh))
        return kh, vh

    def decode(self, q: np.ndarray, sm: float, keep_groups: int = 0, want_logits: bool = False):
        """q: fp32 [U, G, d].  Returns (out fp64 [U, G, d], mask u8 [U][, logits]); with
        bucket-relative RoPE the masks are u8 [U, rope_buckets] (entries past the buckets
        holding positions stay 0)."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        U, G, d = q.shape
        assert U == self.U and d == self.geo.head_dim
        out = np.zeros((U, G, d), dtype=np.float64)
        mask = np.zeros((U, self.geo.rope_buckets) if self.geo.rope_bucket > 0 else U, dtype=np.uint8)
        logits = np.zeros((U, G, self.len), dtype=np.float64) if want_logits else None
        lib().oracle_decode_attn(*self._cache_args(), _p(self.cent), U, self.len, G, _p(q),
                                 float(sm), int(keep_groups), _p(out), _p(mask), _p(logits))
        if want_logits:
            return out, mask, logits
        return out, mask


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))
