"""GPU parity on the eight decode workloads at their full sizes, in the launch
configuration the bench times.

The whole cache is built on the GPU; the oracle re-encodes sampled sequences and must match
their packed bytes bit for bit, then decodes them (outputs within 2e-3 of the row norm,
masks exact).  Inputs are drawn on the GPU by the seeded generators and the sampled
sequences are copied to the host, so both sides see the same values.
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_kvq_amd import binding as B
from bit_kv_cache_kvq_amd import synth
from gpu_util import compare_buffers, compare_outputs, note, oracle_geo, to_f32_np

pytestmark = pytest.mark.gpu


def _build(w, extra=0):
    cap = w.capacity(extra)
    c = B.Cache(w.batch, w.n_kv_heads, w.head_dim, cap, n_sink=w.n_sink, k_format=w.k_format,
                k_hadamard=w.k_hadamard, k_ch0_bf16=w.k_ch0_bf16, v_format=w.v_format, v_clip=w.v_clip,
                n_recent=w.n_recent, rope_bucket=w.rope_bucket, rope_table=synth.rope_table(w, cap),
                qjl_signs=synth.qjl_signs(w.head_dim) if w.v_format == 2 else None)
    k, v = synth.prefill(w, device="cuda")
    note(f"workload {w.name}: prefill {tuple(k.shape)} {k.dtype}, capacity {cap}")
    c.append(k, v)
    torch.cuda.synchronize()
    return c, k, v


def _oracle_for(oracle_mod, c, w, k, v, seqs):
    """Oracle caches for the sampled sequences (units of one sequence are consecutive)."""
    H = w.n_kv_heads
    out = {}
    for b in seqs:
        oc = oracle_geo(oracle_mod, c, units=H)
        oc.append(to_f32_np(k[b]), to_f32_np(v[b]))
        compare_buffers(c, oc, b * H, (b + 1) * H, what=f"{w.name} seq {b}")
        out[b] = oc
    note(f"  packed bytes identical for sequences {list(seqs)}")
    return out


def _check_decode(c, w, ocs, q, what):
    out, mask = c.decode(q, w.sm_scale, w.keep_groups)
    torch.cuda.synchronize()
    H, G, d = w.n_kv_heads, w.group, w.head_dim
    worst = 0.0
    for b, oc in ocs.items():
        qb = to_f32_np(q[b]).reshape(H, G, d)
        ref, rmask = oc.decode(qb, w.sm_scale, w.keep_groups)
        np.testing.assert_array_equal(mask.view(-1, c.rope_buckets)[b * H:(b + 1) * H].cpu().numpy()
                                      .reshape(rmask.shape), rmask)
        worst = max(worst, compare_outputs(out[b], ref, f"{what} seq {b}"))
    note(f"  {what}: outputs within tolerance, worst err/||o|| = {worst:.2e}")
    return out, mask


@pytest.mark.parametrize("wid", [1, 2])
def test_small_workloads_full(oracle_mod, wid):
    w = synth.WORKLOADS[wid]
    c, k, v = _build(w)
    ocs = _oracle_for(oracle_mod, c, w, k, v, range(w.batch))
    q = synth.query(w, 0, device="cuda")
    _check_decode(c, w, ocs, q, f"cfg{wid}")


def test_workload3_wht_lloyd4(oracle_mod):
    w = synth.WORKLOADS[3]
    c, k, v = _build(w)
    ocs = _oracle_for(oracle_mod, c, w, k, v, [0, w.batch - 1])
    _check_decode(c, w, ocs, synth.query(w, 0, device="cuda"), "cfg3")


def test_workload4_pruned_128k(oracle_mod):
    w = synth.WORKLOADS[4]
    c, k, v = _build(w)
    ocs = _oracle_for(oracle_mod, c, w, k, v, [0, w.batch - 1])
    q = synth.query(w, 0, device="cuda")
    _, mask = _check_decode(c, w, ocs, q, "cfg4")
    # masks of every unit depend on the queries only: check all of them
    qn = to_f32_np(q).reshape(w.units, w.group, w.head_dim)
    ref = [oracle_mod.prune_mask(qn[u], w.keep_groups) for u in range(w.units)]
    np.testing.assert_array_equal(mask.cpu().numpy(), np.array(ref, np.uint8))
    assert all(bin(int(m)).count("1") == w.keep_groups for m in ref)


def test_workload6_dualqk_storage_128k(oracle_mod):
    """Dual-QK's storage recipe on the 128K shape: the first 64 and most recent 256 positions
    in BF16, per-token INT2 values clipped to 0.92, INT2 keys with channel 0 in BF16, 5 of 8
    groups kept."""
    w = synth.WORKLOADS[6]
    c, k, v = _build(w)
    ocs = _oracle_for(oracle_mod, c, w, k, v, [0, w.batch - 1])
    _check_decode(c, w, ocs, synth.query(w, 0, device="cuda"), "cfg6")


def test_workload7_rope_buckets_128k(oracle_mod):
    """Workload 6 with bucket-relative RoPE (buckets of 2048 positions, 64 per sequence): one
    query record and mask per bucket, tiles of all buckets in one softmax."""
    w = synth.WORKLOADS[7]
    c, k, v = _build(w)
    ocs = _oracle_for(oracle_mod, c, w, k, v, [0, w.batch - 1])
    _, mask = _check_decode(c, w, ocs, synth.query(w, 0, device="cuda"), "cfg7")
    m = mask.view(-1, c.rope_buckets)[:, :64].cpu().numpy()
    assert len(np.unique(m)) > 1  # the buckets' masks differ


def test_workload8_kqv_values(oracle_mod):
    """The KQV scheme on workload 3's shape: WHT + Lloyd-Max keys, values as rotated 3-bit
    Lloyd-Max codes plus a 1-bit QJL sketch of the residual."""
    w = synth.WORKLOADS[8]
    c, k, v = _build(w)
    ocs = _oracle_for(oracle_mod, c, w, k, v, [0, w.batch - 1])
    _check_decode(c, w, ocs, synth.query(w, 0, device="cuda"), "cfg8")


def test_workload5_append_decode_steps(oracle_mod):
    w = synth.WORKLOADS[5]
    c, k, v = _build(w)
    seqs = [0, w.batch - 1]
    ocs = _oracle_for(oracle_mod, c, w, k, v, seqs)
    del k, v
    H = w.n_kv_heads
    for step in range(w.steps):
        kn, vn = synth.append_tokens(w, step, device="cuda")
        c.append(kn, vn)
        for b in seqs:
            ocs[b].append(to_f32_np(kn[b]), to_f32_np(vn[b]))
        q = synth.query(w, step, device="cuda")
        if step in (0, 31, w.steps - 1):
            torch.cuda.synchronize()
            for b in seqs:
                compare_buffers(c, ocs[b], b * H, (b + 1) * H, what=f"cfg5 step {step} seq {b}")
            _check_decode(c, w, ocs, q, f"cfg5 step {step} (len {c.len})")
        else:
            c.decode(q, w.sm_scale, w.keep_groups)
    assert c.len == w.context + w.steps
