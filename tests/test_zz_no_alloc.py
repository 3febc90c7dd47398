"""The allocation-free decode entry point (kvq_decode_attn_noalloc), called through the C ABI:
on two calls in a row -- the second on a smaller cache -- its outputs and masks equal those
of kvq_decode_attn (bit for bit in the deterministic tile order) and the oracle's within
2e-3 of the row norm; a geometry whose workspace exceeds the library's array is refused."""
import numpy as np
import pytest
import torch

from bit_kv_cache_kvq_amd import binding as B
from bit_kv_cache_kvq_amd import synth
from gpu_util import compare_outputs, note, oracle_geo, to_f32_np

pytestmark = pytest.mark.gpu

SCRATCH = 32 << 20  # KVQ_NOALLOC_SCRATCH_BYTES


def _case(oracle_mod, Bsz, Hkv, T, G, kfmt, ch0, ns, keep, vfmt, nr, rope, seed):
    d = 128
    cap = max(256, (T + 255) // 256 * 256)
    note(f"noalloc case B={Bsz} Hkv={Hkv} T={T} G={G} kfmt={kfmt} ch0={ch0} ns={ns} keep={keep} vfmt={vfmt} "
         f"nr={nr} rope={rope}")
    c = B.Cache(Bsz, Hkv, d, cap, n_sink=ns, k_format=kfmt, k_ch0_bf16=ch0, v_format=vfmt, v_clip=0.92,
                n_recent=nr, rope_bucket=rope, rope_table=synth.rope_anchor_table(d, rope, cap) if rope else None)
    k = synth.student_t3((Bsz, Hkv, T, d), "cpu", seed, 400, 0).to(torch.bfloat16)
    v = synth.normal((Bsz, Hkv, T, d), "cpu", seed, 400, 1).to(torch.bfloat16)
    c.append(k.cuda(), v.cuda())
    q = synth.normal((Bsz, Hkv * G, d), "cpu", seed, 400, 2).to(torch.bfloat16).cuda()
    need = c.noalloc_scratch_bytes(Hkv * G)
    assert 0 < need <= SCRATCH
    sm = 1.0 / np.sqrt(d)
    o_ws, m_ws = c.decode(q, sm, keep)
    o_na, m_na = c.decode_noalloc(q, sm, keep)
    torch.cuda.synchronize()
    assert torch.equal(o_ws, o_na), "allocation-free outputs differ from the workspace entry point's"
    assert torch.equal(m_ws, m_na)
    oc = oracle_geo(oracle_mod, c)
    oc.append(to_f32_np(k).reshape(Bsz * Hkv, T, d), to_f32_np(v).reshape(Bsz * Hkv, T, d))
    ref, rmask = oc.decode(to_f32_np(q).reshape(Bsz * Hkv, G, d), sm, keep)
    np.testing.assert_array_equal(m_na.cpu().numpy().reshape(rmask.shape), rmask)
    worst = compare_outputs(o_na, ref, "noalloc")
    note(f"  equal to kvq_decode_attn; worst err/||o|| = {worst:.2e}; scratch {need} bytes")


def test_noalloc_matches_workspace_entry_point(oracle_mod):
    B.set_deterministic(True)
    try:
        # larger first (wave teams, partial states), then a smaller cache of other formats
        _case(oracle_mod, 4, 4, 3000, 4, 0, 1, 4, 5, 0, 0, 0, 1)
        _case(oracle_mod, 2, 2, 700, 4, 0, 0, 0, 0, 1, 16, 128, 2)
    finally:
        B.set_deterministic(False)


def test_noalloc_default_tile_order_and_repeats(oracle_mod):
    """Default (run-time) tile order: repeated calls on the shared array stay within tolerance."""
    d, cap = 128, 5120
    c = B.Cache(1, 2, d, cap, n_sink=4, k_format=0, k_ch0_bf16=1)
    k = synth.normal((1, 2, 5000, d), "cpu", 3, 400, 0).to(torch.bfloat16)
    v = synth.normal((1, 2, 5000, d), "cpu", 3, 400, 1).to(torch.bfloat16)
    c.append(k.cuda(), v.cuda())
    q = synth.normal((1, 8, d), "cpu", 3, 400, 2).to(torch.bfloat16).cuda()
    oc = oracle_geo(oracle_mod, c)
    oc.append(to_f32_np(k).reshape(2, 5000, d), to_f32_np(v).reshape(2, 5000, d))
    ref, _ = oc.decode(to_f32_np(q).reshape(2, 4, d), 1 / np.sqrt(d), 0)
    for _ in range(3):
        out, _ = c.decode_noalloc(q, 1 / np.sqrt(d))
        torch.cuda.synchronize()
        compare_outputs(out, ref, "noalloc repeat")


def test_noalloc_refuses_oversize_workspace():
    """More partial states than the array holds: KVQ_ERR_WORKSPACE before anything is enqueued."""
    c = B.Cache(512, 8, 128, 256, k_format=0)  # 4096 units: their query records alone exceed it
    n = c.noalloc_scratch_bytes(64)           # G = 8
    assert n > SCRATCH
    q = torch.zeros(512, 64, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full((512, 64, 128), 7.0, device="cuda")
    with pytest.raises(B.KvqError) as e:
        c.decode_noalloc(q, 0.088, out=out)
    assert e.value.status == B.KVQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing was launched
