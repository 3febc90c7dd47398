"""GPU parity at the edges of the input contract.

* Sharp queries (Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV Caches, sec. 1
  and 3.2): 1-4 query channels scaled x100 / x1000 over key channels scaled down by the
  same factor, for every key format, with and without pruning.
* Caches far from unit scale: keys and values x1e-4, keys x1e4 with the query x1e-4, values
  x1.2e4 (group INT4, per-token INT2 with ranges above 6e4, Dual-QK sec. B.2) and KQV
  values with norms above 1e4 (KV-quantisation statistics, scheme KQV).
* Encoder inputs crafted to hit rint ties at k + 1/2, fp16-subnormal scales and zero points,
  signed-zero minima, degenerate groups, a rotated coordinate exactly on a Lloyd-Max
  threshold, and fp32 -> bf16 rounding ties of sinks, recent-window rows and channel 0.

Packed bytes must equal the oracle's bit for bit; outputs within 2e-3 of the oracle row norm.
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_kvq_amd import binding as B
from bit_kv_cache_kvq_amd import synth
from gpu_util import compare_buffers, compare_outputs, note, oracle_geo, to_f32_np

pytestmark = pytest.mark.gpu

LIMIT = 59000.0  # inputs stay inside |x| < 6e4


def _check(oracle_mod, k, v, q, *, kfmt=0, rot=0, ch0=0, keep=0, vfmt=0, vclip=0.92, ns=0, nr=0, what=""):
    """k, v [B, Hkv, T, d], q [B, Hq, d] (torch, CPU, fp32 or bf16): append in two calls,
    compare packed bytes, decode, compare outputs and masks."""
    Bsz, Hkv, T, d = k.shape
    G = q.shape[1] // Hkv
    cap = max(256, (T + 255) // 256 * 256)
    note(f"case {what}: d={d} T={T} G={G} kfmt={kfmt} rot={rot} ch0={ch0} keep={keep} vfmt={vfmt} ns={ns} nr={nr} "
         f"dtype={k.dtype}")
    c = B.Cache(Bsz, Hkv, d, cap, n_sink=ns, k_format=kfmt, k_hadamard=rot, k_ch0_bf16=ch0, v_format=vfmt,
                v_clip=vclip, n_recent=nr, qjl_signs=synth.qjl_signs(d) if vfmt == B.V_KQV else None)
    oc = oracle_geo(oracle_mod, c)
    cut = [0, T // 3, T] if T > 3 else [0, T]
    for a, b in zip(cut[:-1], cut[1:]):
        kc, vc = k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous()
        c.append(kc.cuda(), vc.cuda())
        oc.append(to_f32_np(kc).reshape(Bsz * Hkv, b - a, d), to_f32_np(vc).reshape(Bsz * Hkv, b - a, d))
    torch.cuda.synchronize()
    compare_buffers(c, oc, what=what)
    sm = 1.0 / np.sqrt(d)
    out, mask = c.decode(q.cuda(), sm, keep)
    torch.cuda.synchronize()
    ref, rmask = oc.decode(to_f32_np(q).reshape(Bsz * Hkv, G, d), sm, keep)
    np.testing.assert_array_equal(mask.cpu().numpy().reshape(rmask.shape), rmask)
    worst = compare_outputs(out, ref, what)
    note(f"  ok, worst err/||o|| = {worst:.2e}")
    return worst


def _draw(seed, Bsz, Hkv, T, d, G, dist="normal"):
    f = synth.student_t3 if dist == "t3" else synth.normal
    k = f((Bsz, Hkv, T, d), "cpu", seed, 300, 0)
    v = f((Bsz, Hkv, T, d), "cpu", seed, 300, 1)
    q = synth.normal((Bsz, Hkv * G, d), "cpu", seed, 300, 2)
    return k, v, q


# ---------------------------------------------------------------- sharp query channels
@pytest.mark.parametrize("kfmt,rot,ch0", [(0, 0, 1), (0, 0, 0), (1, 0, 0), (2, 1, 0), (2, 0, 0)])
@pytest.mark.parametrize("factor", [100.0, 1000.0])
@pytest.mark.parametrize("keep", [0, 5])
def test_sharp_query_channels(oracle_mod, kfmt, rot, ch0, factor, keep):
    d, G = 128, 4
    for n, dist, seed in ((1, "normal", 1), (4, "t3", 2)):
        chans = [7, 45, 83, 121][:n]
        k, v, q = _draw(seed, 1, 2, 1500, d, G, dist)
        k[..., chans] /= factor
        q[..., chans] *= factor
        _check(oracle_mod, k.to(torch.bfloat16), v.to(torch.bfloat16), q.to(torch.bfloat16), kfmt=kfmt, rot=rot,
               ch0=ch0, keep=keep, what=f"sharp x{factor:g} on {n} channels ({dist} keys)")


def test_sharp_query_in_one_head_with_sinks_and_window(oracle_mod):
    """Only one head of the GQA group is sharp; BF16 sinks and a recent window take the same
    query; per-token INT2 values."""
    d, G = 128, 4
    k, v, q = _draw(5, 2, 2, 900, d, G, "t3")
    k[..., 45] /= 300.0
    q[:, 1, 45] *= 300.0
    _check(oracle_mod, k, v, q, kfmt=0, ch0=1, keep=5, vfmt=1, ns=4, nr=64, what="one sharp head")


# ---------------------------------------------------------------- caches far from unit scale
@pytest.mark.parametrize("vfmt", [0, 1, 2])
@pytest.mark.parametrize("kfmt,rot,ch0", [(0, 0, 1), (1, 0, 0), (2, 1, 0)])
def test_scaled_caches(oracle_mod, vfmt, kfmt, rot, ch0):
    d, G = 128, 4
    k, v, q = _draw(7, 1, 2, 1100, d, G)
    # keys and values x1e-4 (fp16-subnormal scales and zero points, tiny value weights)
    _check(oracle_mod, k * 1e-4, v * 1e-4, q, kfmt=kfmt, rot=rot, ch0=ch0, vfmt=vfmt, ns=4,
           what="K, V x1e-4")
    # large keys with the query scaled down as much (logits of unit size from large scales
    # and zero points); Lloyd-Max keys x1e3, as their fp16 norm is the key's L2 norm
    ks = 1e3 if kfmt == 2 else 1e4
    _check(oracle_mod, (k * ks).clamp(-LIMIT, LIMIT), v, q / ks, kfmt=kfmt, rot=rot, ch0=ch0, vfmt=vfmt,
           what=f"K x{ks:g}, q x{1 / ks:g}")
    # large values: INT4 groups and per-token INT2 (ranges beyond 6e4) x1.2e4; KQV x1000
    # (norms ~1.1e4: the residual norm stays an fp16)
    vs = 1000.0 if vfmt == 2 else 1.2e4
    _check(oracle_mod, k, (v * vs).clamp(-LIMIT, LIMIT), q * 3.0, kfmt=kfmt, rot=rot, ch0=ch0, vfmt=vfmt,
           vclip=0.92, ns=2, nr=32, what=f"V x{vs:g}")


def test_token_int2_values_near_the_fp16_limit(oracle_mod):
    """Per-token INT2 values whose every token spans about [-5.9e4, 5.9e4]: scales near 3.6e4."""
    d, G = 128, 4
    k, v, q = _draw(9, 2, 1, 700, d, G)
    v = torch.sign(v) * LIMIT * (0.5 + 0.5 * torch.rand(v.shape, generator=torch.Generator().manual_seed(3)))
    v[..., 0] = LIMIT
    v[..., 1] = -LIMIT
    _check(oracle_mod, k, v, q * 4.0, kfmt=0, ch0=1, vfmt=1, vclip=1.0, what="INT2 values, range 1.18e5")
    _check(oracle_mod, k, v, q * 4.0, kfmt=0, ch0=1, vfmt=1, vclip=0.92, what="INT2 values, clipped 0.92")


def test_value_scales_spanning_many_binades(oracle_mod):
    """Value groups from 1e-3 to 1e4 in one sequence: the value-weight exponent adapts (down
    only) and every group still decodes within tolerance; sharp attention on small tokens."""
    d, G = 128, 4
    k, v, q = _draw(11, 1, 2, 1300, d, G)
    scales = 10.0 ** torch.linspace(-3, 4, 1300)
    v = (v * scales[None, None, :, None]).clamp(-LIMIT, LIMIT)
    for vfmt in (0, 1):
        _check(oracle_mod, k, v, q * 4.0, kfmt=1, vfmt=vfmt, what=f"value scales 1e-3..1e4 (vfmt {vfmt})")


# ---------------------------------------------------------------- encoder rounding edges
def _edge_rows(d, T, seed):
    """fp32 rows hitting the encoder's rounding edges, 32-channel groups at a time."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    for t in range(T):
        kind = t % 8
        for g in range(d // 32):
            grp = x[t, 32 * g:32 * (g + 1)]
            if kind == 0:    # INT2 ties: min 0, max 3 (scale 1): values k + 1/2
                grp[:] = rng.choice(np.array([0.5, 1.5, 2.5, 0.0, 3.0], np.float32), 32)
                grp[0], grp[1] = 0.0, 3.0
            elif kind == 1:  # INT4 ties: min 0, max 15 (scale 1)
                grp[:] = rng.integers(0, 15, 32).astype(np.float32) + 0.5
                grp[0], grp[1] = 0.0, 15.0
            elif kind == 2:  # fp16-subnormal scale and zero point
                grp[:] = (1e-6 + rng.random(32) * 9e-6).astype(np.float32)
            elif kind == 3:  # signed-zero minimum
                grp[:] = np.abs(grp)
                grp[5] = -0.0
            elif kind == 4:  # degenerate group
                grp[:] = np.float32(1.25)
            elif kind == 5:  # fp32 -> bf16 ties (low half exactly 0x8000), both parities
                b = rng.integers(0x3F00, 0x4100, 32).astype(np.uint32)
                grp[:] = ((b << 16) | 0x8000).view(np.float32)
            elif kind == 6:  # ties of the clipped per-token range and channel 0 extremes
                grp[:] = np.float32(0.75) * rng.integers(-4, 5, 32).astype(np.float32)
        if kind == 5:
            x[t, 0] = np.uint32(0x3FC18000).view(np.float32)  # channel 0 itself on a bf16 tie
    return x


@pytest.mark.parametrize("kfmt,ch0,vfmt,vclip", [(0, 1, 0, 0.92), (1, 0, 1, 1.0), (0, 0, 1, 0.92)])
def test_encoder_rounding_edges(oracle_mod, kfmt, ch0, vfmt, vclip):
    d, G, T = 128, 2, 520
    k = torch.from_numpy(_edge_rows(d, T, 1)).reshape(1, 1, T, d)
    v = torch.from_numpy(_edge_rows(d, T, 2)).reshape(1, 1, T, d)
    q = synth.normal((1, G, d), "cpu", 13, 300, 2)
    _check(oracle_mod, k, v, q, kfmt=kfmt, ch0=ch0, vfmt=vfmt, vclip=vclip, ns=8, nr=16,
           what="encoder edges")


def test_lloyd_max_codes_on_thresholds(oracle_mod):
    """Unrotated Lloyd-Max keys whose norm rounds to exactly 1 and whose coordinates sit exactly
    on the 15 decision thresholds (ties go to the lower code) or on the centroids."""
    d, G, T = 128, 4, 300
    cent, thr = B.codebook_gaussian(4)
    thr = np.asarray(thr, np.float32)
    cent = np.asarray(cent, np.float32)
    rng = np.random.default_rng(4)
    x = np.zeros((T, d), np.float32)
    for t in range(T):
        pick = thr if t % 2 == 0 else cent
        head = rng.permutation(np.concatenate([pick, -pick]))[:30].astype(np.float32)
        rest = d - head.size
        fill = np.float32(np.sqrt(max(d - float(np.sum(head.astype(np.float64) ** 2)), rest * 0.25) / rest))
        row = np.concatenate([head, fill * rng.choice(np.array([-1, 1], np.float32), rest)])
        x[t] = row[rng.permutation(d)]
    k = torch.from_numpy(x).reshape(1, 1, T, d)
    v = synth.normal((1, 1, T, d), "cpu", 4, 300, 1)
    q = synth.normal((1, G, d), "cpu", 4, 300, 2)
    _check(oracle_mod, k, v, q, kfmt=2, rot=0, what="Lloyd-Max thresholds")
