"""GPU parity of the HIP path against the CPU oracle on small and ragged shapes.

Packed bytes must match bit for bit; attention outputs within 2e-3 of the oracle row norm;
pruning masks exactly.  Inputs come from the seeded generators (CPU draws copied to the
GPU), so both sides see identical values.
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_kvq_amd import binding as B
from bit_kv_cache_kvq_amd import synth
from gpu_util import compare_buffers, compare_outputs, note, oracle_geo, to_f32_np

pytestmark = pytest.mark.gpu


def _inputs(seed, Bsz, Hkv, T, d, dist="normal", dtype=torch.bfloat16, outliers=()):
    shape = (Bsz, Hkv, T, d)
    if dist == "t3":
        k = synth.student_t3(shape, "cpu", seed, 100, 0)
        v = synth.student_t3(shape, "cpu", seed, 100, 1)
    else:
        k = synth.normal(shape, "cpu", seed, 100, 0)
        v = synth.normal(shape, "cpu", seed, 100, 1)
    for ch, f in outliers:
        k[..., ch] *= f
    return k.to(dtype), v.to(dtype)


def _run(oracle_mod, *, d=128, kfmt=0, rot=0, ch0=0, ns=0, T=300, G=4, Hkv=2, Bsz=2, keep=0,
         dtype=torch.bfloat16, chunks=None, dist="normal", seed=0, cap=None, q_scale=1.0, outliers=(),
         vfmt=0, vclip=0.92, nr=0, rope=0):
    cap = cap or max(256, (T + 255) // 256 * 256)
    note(f"case d={d} kfmt={kfmt} rot={rot} ch0={ch0} ns={ns} T={T} G={G} Hkv={Hkv} B={Bsz} keep={keep} "
         f"dtype={dtype} chunks={chunks} dist={dist} vfmt={vfmt} vclip={vclip} nr={nr} rope={rope}")
    c = B.Cache(Bsz, Hkv, d, cap, n_sink=ns, k_format=kfmt, k_hadamard=rot, k_ch0_bf16=ch0,
                v_format=vfmt, v_clip=vclip, n_recent=nr, rope_bucket=rope,
                rope_table=synth.rope_anchor_table(d, rope, cap) if rope else None,
                qjl_signs=synth.qjl_signs(d, seed) if vfmt == B.V_KQV else None)
    oc = oracle_geo(oracle_mod, c)
    k, v = _inputs(seed, Bsz, Hkv, T, d, dist, dtype, outliers)
    chunks = chunks or [T]
    assert sum(chunks) == T
    t = 0
    for n in chunks:
        kc, vc = k[:, :, t:t + n].contiguous(), v[:, :, t:t + n].contiguous()
        c.append(kc.cuda(), vc.cuda())
        oc.append(to_f32_np(kc).reshape(Bsz * Hkv, n, d), to_f32_np(vc).reshape(Bsz * Hkv, n, d))
        t += n
    torch.cuda.synchronize()
    assert c.len == T == oc.len
    compare_buffers(c, oc, what="append")
    q = (synth.normal((Bsz, Hkv * G, d), "cpu", seed, 100, 2) * q_scale).to(dtype)
    sm = 1.0 / np.sqrt(d)
    out, mask = c.decode(q.cuda(), sm, keep)
    torch.cuda.synchronize()
    ref, rmask = oc.decode(to_f32_np(q).reshape(Bsz * Hkv, G, d), sm, keep)
    np.testing.assert_array_equal(mask.cpu().numpy().reshape(rmask.shape), rmask)
    worst = compare_outputs(out, ref, "decode")
    note(f"  ok, worst err/||o|| = {worst:.2e}")
    return c, oc, q, out


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 255, 256, 257, 1000])
def test_asym2_ch0_ragged_lengths(oracle_mod, T):
    _run(oracle_mod, kfmt=0, ch0=1, T=T)


@pytest.mark.parametrize("d,kfmt,rot,ch0,G,dtype", [
    (64, 0, 0, 1, 1, torch.float32),
    (64, 1, 0, 0, 2, torch.bfloat16),
    (64, 2, 1, 0, 4, torch.bfloat16),
    (64, 2, 0, 0, 8, torch.float32),
    (128, 1, 0, 1, 1, torch.float32),
    (128, 2, 1, 0, 4, torch.bfloat16),
    (128, 2, 0, 0, 2, torch.bfloat16),
    (128, 0, 0, 0, 8, torch.bfloat16),
    (128, 1, 0, 0, 4, torch.bfloat16),
])
def test_formats_and_groups(oracle_mod, d, kfmt, rot, ch0, G, dtype):
    _run(oracle_mod, d=d, kfmt=kfmt, rot=rot, ch0=ch0, G=G, dtype=dtype, T=777)


@pytest.mark.parametrize("keep", [1, 3, 5, 7, 8])
@pytest.mark.parametrize("kfmt,rot,ch0", [(0, 0, 1), (2, 1, 0), (1, 0, 0)])
def test_pruning(oracle_mod, keep, kfmt, rot, ch0):
    _run(oracle_mod, kfmt=kfmt, rot=rot, ch0=ch0, keep=keep, T=600)


@pytest.mark.parametrize("ns,T", [(4, 300), (3, 3), (4, 2), (64, 64), (64, 70), (1, 257), (5, 1000)])
def test_sinks(oracle_mod, ns, T):
    _run(oracle_mod, kfmt=0, ns=ns, T=T, dist="t3", keep=0)


def test_sinks_with_pruning_and_rotation(oracle_mod):
    _run(oracle_mod, kfmt=2, rot=1, ns=4, T=500, keep=4)
    _run(oracle_mod, kfmt=0, ch0=1, ns=8, T=500, keep=3, d=64, G=2)


def test_incremental_appends_match_bulk(oracle_mod):
    _run(oracle_mod, kfmt=0, ch0=1, ns=4, T=300, chunks=[5, 1, 1, 100, 1, 192])
    _run(oracle_mod, kfmt=2, rot=1, T=261, chunks=[256, 1, 1, 1, 1, 1])


def test_heavy_tails_and_outliers(oracle_mod):
    _run(oracle_mod, kfmt=0, ch0=1, T=2000, dist="t3", outliers=((7, 8.0), (45, 8.0)))
    _run(oracle_mod, kfmt=0, T=2000, q_scale=6.0)  # sharp attention


def test_zero_length_and_sink_only(oracle_mod):
    c = B.Cache(2, 2, 128, 256, n_sink=4)
    q = torch.randn(2, 8, 128, device="cuda")
    out, _ = c.decode(q, 0.088)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    _run(oracle_mod, ns=4, T=4)


def test_split_invariance_and_determinism(oracle_mod):
    c, oc, q, out0 = _run(oracle_mod, kfmt=0, ch0=1, T=5000, Bsz=1, Hkv=2, G=4)
    qg = q.cuda()
    ref, _ = oc.decode(to_f32_np(q).reshape(2, 4, 128), 1 / np.sqrt(128))
    try:
        for det in (True, False):
            B.set_deterministic(det)
            for tps in (1, 2, 3, 7, 20):
                B.set_split_tiles(tps)
                note(f"  deterministic {det}, split tiles {tps}: {c.splits(8)} waves")
                o1, _ = c.decode(qg, 1 / np.sqrt(128))
                o2, _ = c.decode(qg, 1 / np.sqrt(128))
                torch.cuda.synchronize()
                if det:
                    assert torch.equal(o1, o2), "run-to-run difference"
                compare_outputs(o1, ref, f"split tiles {tps}")
                compare_outputs(o2, ref, f"split tiles {tps}")
    finally:
        B.set_split_tiles(0)
        B.set_deterministic(False)


@pytest.mark.parametrize("kfmt,rot,ch0,keep,G,d", [(0, 0, 0, 0, 2, 128), (2, 1, 0, 3, 4, 128),
                                                   (1, 0, 1, 5, 1, 64), (0, 0, 1, 2, 8, 64)])
def test_wave_teams_across_units(oracle_mod, kfmt, rot, ch0, keep, G, d):
    # 16 short sequences (3 tiles each): from one wave per tile (every tile a member's
    # first) down to one wave per unit; in between, teams of 1-2 waves where the unit's
    # counter hands out the third tile
    c, oc, q, out0 = _run(oracle_mod, d=d, kfmt=kfmt, rot=rot, ch0=ch0, keep=keep, ns=4, T=300, Bsz=4,
                          Hkv=4, G=G, dist="t3")
    qg = q.cuda()
    sm = 1 / np.sqrt(d)
    ref, _ = oc.decode(to_f32_np(q).reshape(16, G, d), sm, keep)
    try:
        for tps in (1, 2, 4, 5, 7, 13, 48, 1000):
            B.set_split_tiles(tps)
            note(f"  tiles per wave {tps}: {c.splits(4 * G)} waves")
            o1, _ = c.decode(qg, sm, keep)
            torch.cuda.synchronize()
            compare_outputs(o1, ref, f"tiles per wave {tps}")
    finally:
        B.set_split_tiles(0)


def test_teams_drawing_many_tiles(oracle_mod):
    # 4 sequences of 40 tiles: teams of 2..40 waves draw most tiles from the unit counters
    # in whatever order the waves ask; every order gives the oracle's output
    c, oc, q, _ = _run(oracle_mod, kfmt=0, ch0=1, ns=4, T=5000, Bsz=2, Hkv=2, G=4, dist="t3")
    qg = q.cuda()
    sm = 1 / np.sqrt(128)
    ref, _ = oc.decode(to_f32_np(q).reshape(4, 4, 128), sm, 0)
    try:
        for tps in (1, 2, 3, 7, 20):
            B.set_split_tiles(tps)
            note(f"  tiles per wave {tps}: {c.splits(16)} waves")
            for _ in range(3):
                o1, _ = c.decode(qg, sm, 0)
                torch.cuda.synchronize()
                compare_outputs(o1, ref, f"tiles per wave {tps}")
    finally:
        B.set_split_tiles(0)


def test_keep_all_equals_no_pruning(oracle_mod):
    # (in the fixed tile order: by default the order tiles are drawn in changes the last bits)
    B.set_deterministic(True)
    try:
        for T in (700, 5000):
            c, oc, q, out0 = _run(oracle_mod, kfmt=0, ch0=1, T=T, keep=0)
            o8, m8 = c.decode(q.cuda(), 1 / np.sqrt(128), 8)
            o9, _ = c.decode(q.cuda(), 1 / np.sqrt(128), 100)
            torch.cuda.synchronize()
            assert torch.equal(out0, o8) and torch.equal(out0, o9)
            assert torch.all(m8 == 0xFF)
    finally:
        B.set_deterministic(False)


def test_decode_leaves_cache_unchanged(oracle_mod):
    c, oc, q, _ = _run(oracle_mod, kfmt=0, ch0=1, T=400, keep=5)
    before = {k: v.clone() for k, v in c.buffers.items()}
    c.decode(q.cuda(), 0.088, 5)
    c.decode(q.cuda(), 0.088, 2)
    torch.cuda.synchronize()
    for k, v in c.buffers.items():
        assert torch.equal(before[k], v), k


def test_decode_event_hook(oracle_mod):
    # the library records the caller's events around the main decode kernel only
    c, oc, q, out0 = _run(oracle_mod, kfmt=0, T=3000, Bsz=2, Hkv=2)
    e0, e1, c0, c1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    for e in (e0, e1):
        e.record()
    torch.cuda.synchronize()
    try:
        B.set_decode_events(e0, e1)
        c0.record()
        out, _ = c.decode(q.cuda(), 1 / np.sqrt(128))
        c1.record()
        torch.cuda.synchronize()
    finally:
        B.set_decode_events()
    kern, call = e0.elapsed_time(e1), c0.elapsed_time(c1)
    note(f"  decode kernel {kern * 1e3:.1f} us of a {call * 1e3:.1f} us call")
    assert 0 < kern <= call
    assert torch.equal(out, out0)


# per-token INT2 values with a clipping ratio (Dual-QK sec. B.2)
@pytest.mark.parametrize("d,kfmt,rot,ch0,G,keep,ns,T,vclip", [
    (128, 0, 0, 1, 4, 5, 4, 300, 0.92),
    (128, 0, 0, 0, 4, 0, 0, 1, 0.92),
    (128, 0, 0, 1, 4, 0, 64, 1000, 0.92),
    (128, 2, 1, 0, 4, 3, 0, 257, 0.92),
    (128, 1, 0, 0, 8, 0, 2, 129, 1.0),
    (128, 0, 0, 0, 1, 0, 0, 65, 0.5),
    (64, 0, 0, 1, 2, 2, 3, 255, 0.92),
    (64, 2, 0, 0, 8, 0, 0, 384, 0.92),
])
def test_token_int2_values(oracle_mod, d, kfmt, rot, ch0, G, keep, ns, T, vclip):
    _run(oracle_mod, d=d, kfmt=kfmt, rot=rot, ch0=ch0, G=G, keep=keep, ns=ns, T=T, vfmt=1, vclip=vclip,
         chunks=[T // 3, T - T // 3] if T > 3 else None)


def test_token_int2_values_teams_and_heavy_tails(oracle_mod):
    """Long context on few units (wave teams, striped), Student-t3 values, across calls."""
    _run(oracle_mod, d=128, kfmt=0, ch0=1, G=4, keep=5, ns=4, T=9000, Hkv=1, Bsz=1, dist="t3", vfmt=1)
    for tps in (1, 3):
        B.set_split_tiles(tps)
        try:
            _run(oracle_mod, d=128, kfmt=0, G=4, T=4000, Hkv=2, Bsz=1, vfmt=1, seed=3)
        finally:
            B.set_split_tiles(0)


# recent BF16 window (Dual-QK sec. 3.3 / 4.1; past-only quantization)
@pytest.mark.parametrize("d,kfmt,rot,ch0,G,keep,ns,T,nr,vfmt,chunks", [
    (128, 0, 0, 1, 4, 5, 64, 1000, 256, 1, [300, 1, 699]),
    (128, 0, 0, 0, 4, 0, 0, 300, 1, 0, [299, 1]),
    (128, 0, 0, 1, 4, 0, 4, 10, 16, 0, [3, 7]),
    (128, 1, 0, 0, 4, 0, 2, 1000, 100, 0, None),
    (128, 2, 1, 0, 4, 3, 0, 700, 256, 1, [200, 500]),
    (64, 0, 0, 1, 8, 2, 3, 333, 64, 0, [100, 233]),
    (64, 2, 0, 0, 2, 0, 0, 130, 130, 1, [60, 70]),
    # more than 8 sinks (a chunk workgroup of their own) with a window, under G = 8, 1 and 4:
    # the chunk's rows split over 8, 1 and 4 waves
    (128, 0, 0, 1, 8, 3, 16, 500, 96, 0, [250, 250]),
    (128, 1, 0, 0, 1, 0, 12, 300, 70, 1, [150, 150]),
    (64, 0, 0, 0, 4, 2, 9, 200, 33, 0, None),
])
def test_recent_window(oracle_mod, d, kfmt, rot, ch0, G, keep, ns, T, nr, vfmt, chunks):
    _run(oracle_mod, d=d, kfmt=kfmt, rot=rot, ch0=ch0, G=G, keep=keep, ns=ns, T=T, nr=nr, vfmt=vfmt,
         chunks=chunks, dtype=torch.float32 if d == 64 else torch.bfloat16)


def test_recent_window_single_token_steps(oracle_mod):
    """One append per step (the decode-time pattern): every step evicts the oldest window
    position; decoded after the last step, and with teams drawing tiles."""
    _run(oracle_mod, d=128, kfmt=0, G=4, ns=4, T=2100, nr=256, Hkv=1, Bsz=2, chunks=[2000] + [1] * 100,
         dist="t3", vfmt=1)


# bucket-relative RoPE (Dual-QK sec. 3.4 / C.4): keys stored relative to their bucket's anchor,
# one query record and mask per bucket, one softmax over all buckets
@pytest.mark.parametrize("d,kfmt,rot,ch0,G,keep,ns,T,nr,vfmt,rope,chunks", [
    (128, 0, 0, 1, 4, 5, 4, 1000, 0, 0, 128, [999, 1]),
    (128, 0, 0, 1, 4, 5, 64, 1100, 256, 1, 256, [700, 1, 399]),
    (128, 0, 0, 0, 4, 0, 0, 700, 0, 0, 128, None),
    (128, 1, 0, 0, 8, 3, 2, 520, 0, 0, 128, [257, 263]),
    (128, 2, 1, 0, 4, 6, 0, 900, 0, 0, 256, None),
    (128, 2, 0, 0, 2, 0, 0, 300, 100, 0, 128, [150, 150]),
    (64, 0, 0, 1, 1, 3, 3, 640, 200, 0, 128, [300, 340]),
    (64, 2, 1, 0, 8, 2, 0, 333, 0, 1, 1024, None),
    (128, 0, 0, 1, 8, 4, 12, 900, 150, 1, 256, [450, 450]),
])
def test_rope_buckets(oracle_mod, d, kfmt, rot, ch0, G, keep, ns, T, nr, vfmt, rope, chunks):
    _run(oracle_mod, d=d, kfmt=kfmt, rot=rot, ch0=ch0, G=G, keep=keep, ns=ns, T=T, nr=nr, vfmt=vfmt, rope=rope,
         chunks=chunks, dtype=torch.float32 if d == 64 else torch.bfloat16)


def test_rope_buckets_teams(oracle_mod):
    """Long context on one unit (wave teams, striped, tiles drawn across buckets), heavy tails,
    a window spanning a bucket edge; and forced splits."""
    _run(oracle_mod, d=128, kfmt=0, ch0=1, G=4, keep=5, ns=4, T=9000, Hkv=1, Bsz=1, dist="t3", vfmt=1, nr=256,
         rope=2048, chunks=[8100, 1, 899])
    for tps in (1, 3):
        B.set_split_tiles(tps)
        try:
            _run(oracle_mod, d=128, kfmt=0, G=4, keep=4, T=4000, Hkv=2, Bsz=1, seed=3, rope=512)
        finally:
            B.set_split_tiles(0)


# KQV values (Statistical Inference ... Inspired by TurboQuant, scheme KQV): rotated 3-bit codes
# plus a 1-bit QJL sketch of the residual; the estimator and the inverse rotation run in the
# decode kernel's flush
@pytest.mark.parametrize("d,kfmt,rot,ch0,G,keep,ns,T,nr,rope,chunks", [
    (128, 2, 1, 0, 4, 0, 0, 1000, 0, 0, None),
    (128, 0, 0, 1, 4, 5, 4, 777, 0, 0, [700, 1, 76]),
    (128, 0, 0, 0, 8, 0, 64, 300, 100, 0, [150, 150]),
    (128, 1, 0, 0, 2, 3, 0, 520, 0, 128, None),
    (128, 0, 0, 1, 1, 0, 2, 257, 0, 0, None),
    (64, 2, 1, 0, 4, 2, 3, 640, 200, 128, [300, 340]),
    (64, 0, 0, 1, 8, 0, 0, 333, 0, 0, None),
])
def test_kqv_values(oracle_mod, d, kfmt, rot, ch0, G, keep, ns, T, nr, rope, chunks):
    _run(oracle_mod, d=d, kfmt=kfmt, rot=rot, ch0=ch0, G=G, keep=keep, ns=ns, T=T, nr=nr, rope=rope, vfmt=B.V_KQV,
         chunks=chunks, dtype=torch.float32 if d == 64 else torch.bfloat16)


def test_kqv_values_teams(oracle_mod):
    """Long context on one unit (teams of waves, partial states combined after the estimator)."""
    _run(oracle_mod, d=128, kfmt=0, G=4, ns=4, T=9000, Hkv=1, Bsz=1, dist="t3", vfmt=B.V_KQV)


@pytest.mark.parametrize("rope,vfmt,nr", [(128, 0, 0), (0, B.V_KQV, 0), (256, B.V_KQV, 16), (128, 1, 3)])
def test_empty_and_short_caches_of_the_newer_formats(oracle_mod, rope, vfmt, nr):
    """len = 0 writes zeros; sink-only, one-quantised-position and window-only caches match
    the oracle with RoPE buckets, KQV values and recent windows."""
    d = 128
    c = B.Cache(2, 2, d, 256, n_sink=4, v_format=vfmt, v_clip=0.92, n_recent=nr, rope_bucket=rope,
                rope_table=synth.rope_anchor_table(d, rope, 256) if rope else None,
                qjl_signs=synth.qjl_signs(d) if vfmt == B.V_KQV else None)
    q = torch.randn(2, 8, d, device="cuda")
    out, _ = c.decode(q, 0.088)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    for T in (1, 4, 5, 4 + nr + 1):
        _run(oracle_mod, ns=4, T=T, rope=rope, vfmt=vfmt, nr=nr, keep=5)
