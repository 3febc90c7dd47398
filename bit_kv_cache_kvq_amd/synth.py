"""Seeded synthetic inputs for the quantized-KV decode workloads.

This module holds no arithmetic of the method: it only draws random keys, values and
queries with the shapes and distributions of the eight workloads, from torch generators
seeded by a stable hash of (seed, workload, tensor, step).  Both the HIP path and the
CPU oracle consume what it produces; nothing here quantizes, rotates or attends.

The pages evaluate on long-context suites and 32-query/8-KV-head, d=128 models
(Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV Caches, sec. 4.1 and 4.4).
No dataset or model is used: these draws stand in for them with the same head layout
and context lengths (4K to 128K).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import torch

# tensor ids inside a workload's seed tuple
T_KEY, T_VALUE, T_QUERY, T_APPEND_K, T_APPEND_V = 0, 1, 2, 3, 4


def seed_of(*parts: int) -> int:
    h = hashlib.blake2b(repr(tuple(int(p) for p in parts)).encode(), digest_size=8)
    return int.from_bytes(h.digest(), "little") & ((1 << 63) - 1)


def _gen(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def normal(shape, device, *parts: int) -> torch.Tensor:
    """fp32 N(0,1) draws."""
    return torch.randn(*shape, generator=_gen(device, *parts), device=device, dtype=torch.float32)


def student_t3(shape, device, *parts: int) -> torch.Tensor:
    """fp32 standard Student-t with 3 degrees of freedom: z / sqrt(chi2_3 / 3)."""
    g = _gen(device, *parts)
    z = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros_like(z)
    for _ in range(3):
        a = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
        chi.add_(a * a)
    return z / torch.sqrt(chi / 3.0)


@dataclass(frozen=True)
class Workload:
    """One decode workload: cache geometry, formats and input distributions."""

    wid: int
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int
    k_format: int  # 0 asym INT2, 1 asym INT4, 2 Lloyd-Max 4-bit
    k_hadamard: int = 0
    k_ch0_bf16: int = 0
    n_sink: int = 0
    keep_groups: int = 0  # 0 = no query-channel pruning
    in_dtype: str = "bf16"  # dtype of keys, values and queries handed to the library
    dist: str = "normal"  # "normal" | "t3"
    key_outliers: tuple = field(default_factory=tuple)  # (channel, factor) pairs on keys
    steps: int = 0  # decode steps, each appending one token per sequence first
    v_format: int = 0  # 0 asym INT4 per 32-channel group, 1 per-token asym INT2 (clipped)
    v_clip: float = 1.0  # clipping ratio of per-token INT2 values
    n_recent: int = 0  # most recent positions kept in BF16 (0: none)
    rope_bucket: int = 0  # bucket-relative RoPE: bucket width (0: off)
    rope_theta: float = 10000.0  # rotary base of the model the inputs stand for

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads

    def capacity(self, extra: int = 0) -> int:
        """Slots per sequence, a multiple of 256 (the decode tile)."""
        need = self.context + self.steps + extra
        return max(256, (need + 255) // 256 * 256)

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5


WORKLOADS = {
    1: Workload(1, "b1_h1_d64_t128_int2ch0_int4_f32", 1, 1, 1, 64, 128, 0, k_ch0_bf16=1,
                in_dtype="f32", key_outliers=((3, 10.0), (17, 10.0))),
    2: Workload(2, "b1_gqa32x8_d128_t4096_int2ch0_int4", 1, 32, 8, 128, 4096, 0, k_ch0_bf16=1,
                key_outliers=((7, 8.0), (45, 8.0), (83, 8.0), (121, 8.0))),
    3: Workload(3, "b16_gqa32x8_d128_t32768_wht_lloyd4_int4", 16, 32, 8, 128, 32768, 2,
                k_hadamard=1),
    4: Workload(4, "b4_gqa32x8_d128_t131072_int2ch0_prune5of8_int4", 4, 32, 8, 128, 131072, 0,
                k_ch0_bf16=1, keep_groups=5),
    5: Workload(5, "b64_gqa32x8_d128_t16384_t3_sink4_int2_int4_append64", 64, 32, 8, 128, 16384,
                0, n_sink=4, dist="t3", steps=64),
    # Dual-QK's storage recipe (sec. 3.3, 4.1, B.2) on the 128K shape: INT2 keys with channel 0
    # in BF16, 5 of 8 query-channel groups kept, the first 64 and the most recent 256 positions
    # in BF16, per-token INT2 values clipped to 0.92 of their range
    6: Workload(6, "b4_gqa32x8_d128_t131072_int2ch0_prune5of8_sink64_recent256_int2tok_clip092", 4, 32, 8,
                128, 131072, 0, k_ch0_bf16=1, n_sink=64, keep_groups=5, v_format=1, v_clip=0.92,
                n_recent=256),
    # workload 6 with bucket-relative RoPE (Dual-QK sec. 3.4, C.4): buckets of 2048 positions,
    # a rotary base of 10^4; keys and queries count as carrying their rotary embedding
    7: Workload(7, "b4_gqa32x8_d128_t131072_int2ch0_prune5of8_sink64_recent256_int2tok_clip092_rope2048", 4,
                32, 8, 128, 131072, 0, k_ch0_bf16=1, n_sink=64, keep_groups=5, v_format=1, v_clip=0.92,
                n_recent=256, rope_bucket=2048),
    # the KQV scheme at the 4-bit budget (KV-quantisation statistics, "Quantisierungsschemata"):
    # WHT + 4-bit Lloyd-Max keys as workload 3, values WHT + 3-bit Lloyd-Max + 1-bit QJL sketch
    8: Workload(8, "b16_gqa32x8_d128_t32768_wht_lloyd4_kqv3qjl1", 16, 32, 8, 128, 32768, 2, k_hadamard=1,
                v_format=2),
}


def rope_table(w: Workload, capacity: int):
    """The model's rotary (cos, sin) at every bucket anchor: float32 [ceil(capacity / w)][d/2][2],
    entry (b, i) for the angle (b * w) * theta^(-2i/d) (computed in fp64, then rounded).  This
    is the model side's positional table, an input like the keys; None without RoPE.

    The keys and queries drawn here are i.i.d. N(0,1) per channel, whose distribution any
    rotation of a channel pair leaves unchanged, so they serve as keys and queries with
    their rotary embedding already applied; nothing here rotates them."""
    if not w.rope_bucket:
        return None
    return rope_anchor_table(w.head_dim, w.rope_bucket, capacity, w.rope_theta)


def qjl_signs(head_dim: int, seed: int = 0):
    """KQV values' random sign diagonal (the sketch's one random draw): uint32 [head_dim / 32],
    bit i set = channel i negated, seeded like every other input."""
    import numpy as np

    g = _gen("cpu", seed, 9000, head_dim)
    bits = torch.randint(0, 2, (head_dim,), generator=g).numpy().astype(np.uint64)
    return (bits.reshape(-1, 32) << np.arange(32, dtype=np.uint64)).sum(1).astype(np.uint32)


def rope_anchor_table(head_dim: int, bucket: int, capacity: int, theta: float = 10000.0):
    """(cos, sin) of the angles (b * bucket) * theta^(-2i/head_dim), b < ceil(capacity /
    bucket), i < head_dim / 2: float32 [buckets][head_dim/2][2] (fp64, then rounded)."""
    import numpy as np

    nb = -(-capacity // bucket)
    half = head_dim // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = (np.arange(nb, dtype=np.float64) * bucket)[:, None] * inv_freq[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def _torch_dtype(w: Workload):
    return torch.float32 if w.in_dtype == "f32" else torch.bfloat16


def _draw(w: Workload, shape, device, tensor_id: int, step: int, seed: int) -> torch.Tensor:
    if w.dist == "t3" and tensor_id != T_QUERY:
        return student_t3(shape, device, seed, w.wid, tensor_id, step)
    return normal(shape, device, seed, w.wid, tensor_id, step)


def _keys(w: Workload, x: torch.Tensor) -> torch.Tensor:
    for ch, f in w.key_outliers:
        x[..., ch] *= f
    return x


def prefill(w: Workload, device="cpu", seed: int = 0, context: int | None = None,
            batch: int | None = None):
    """Keys and values [B, Hkv, T, d] in the workload's input dtype.

    Drawn one sequence at a time so the fp32 temporaries stay bounded."""
    T = w.context if context is None else context
    B = w.batch if batch is None else batch
    dt = _torch_dtype(w)
    k = torch.empty(B, w.n_kv_heads, T, w.head_dim, dtype=dt, device=device)
    v = torch.empty_like(k)
    for b in range(B):
        shape = (w.n_kv_heads, T, w.head_dim)
        k[b] = _keys(w, _draw(w, shape, device, T_KEY, b, seed)).to(dt)
        v[b] = _draw(w, shape, device, T_VALUE, b, seed).to(dt)
    return k, v


def query(w: Workload, step: int = 0, device="cpu", seed: int = 0, batch: int | None = None):
    """Queries [B, Hq, d] for one decode step, N(0,1)."""
    B = w.batch if batch is None else batch
    q = normal((B, w.n_q_heads, w.head_dim), device, seed, w.wid, T_QUERY, step)
    return q.to(_torch_dtype(w))


def append_tokens(w: Workload, step: int, device="cpu", seed: int = 0, batch: int | None = None):
    """One new key/value token per sequence [B, Hkv, 1, d] for decode step `step`."""
    B = w.batch if batch is None else batch
    shape = (B, w.n_kv_heads, 1, w.head_dim)
    dt = _torch_dtype(w)
    k = _keys(w, _draw(w, shape, device, T_APPEND_K, step, seed)).to(dt)
    v = _draw(w, shape, device, T_APPEND_V, step, seed).to(dt)
    return k, v
