"""Save and restore of a quantized cache on the GPU.

A cache's state is its geometry, len and the bytes of its buffers (Cache.state_dict()),
written with torch.save and read back with torch.load(weights_only=True).  In deterministic
mode (each decode wave takes a fixed set of tiles) decoding the restored cache gives the same
bits as decoding the original, and both caches stay byte-identical as appends continue --
the recent window's ring and its evictions included.
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_kvq_amd import binding as B
from bit_kv_cache_kvq_amd import synth
from gpu_util import note

pytestmark = pytest.mark.gpu


def _tokens(seed, Bsz, Hkv, n, d, dtype, step):
    k = synth.student_t3((Bsz, Hkv, n, d), "cpu", seed, 300, step, 0).to(dtype)
    v = synth.normal((Bsz, Hkv, n, d), "cpu", seed, 300, step, 1).to(dtype)
    return k.cuda(), v.cuda()


@pytest.mark.parametrize("name,kw,Bsz,Hkv,G,keep,chunks,more,dtype,where", [
    ("int2 keys, per-token int2 values, sinks, window, rope", dict(k_format=B.K_ASYM2, k_ch0_bf16=1, n_sink=4,
     v_format=B.V_ASYM2_TOKEN, v_clip=0.92, n_recent=256, rope_bucket=128), 2, 2, 4, 5, [700, 1, 299], [37, 1],
     torch.bfloat16, "cuda"),
    ("rotated Lloyd-Max keys, KQV values, window", dict(k_format=B.K_LLOYD4, k_hadamard=1, v_format=B.V_KQV,
     n_recent=100), 2, 1, 8, 0, [600], [1, 1, 1], torch.float32, "cpu"),
    ("int4 keys and values, one long sequence (wave teams)", dict(k_format=B.K_ASYM4), 1, 1, 4, 3, [3000, 5],
     [300], torch.bfloat16, "cuda"),
])
def test_save_restore_decodes_bit_identical(tmp_path, name, kw, Bsz, Hkv, G, keep, chunks, more, dtype, where):
    note(f"case {name}: B={Bsz} Hkv={Hkv} G={G} keep={keep} chunks={chunks} more={more} load to {where}")
    d = 128
    T = sum(chunks) + sum(more)
    cap = (T + 255) // 256 * 256
    extra = {}
    if kw.get("rope_bucket"):
        extra["rope_table"] = synth.rope_anchor_table(d, kw["rope_bucket"], cap)
    if kw.get("v_format") == B.V_KQV:
        extra["qjl_signs"] = synth.qjl_signs(d, 7)
    B.set_deterministic(True)
    try:
        c = B.Cache(Bsz, Hkv, d, cap, **kw, **extra)
        step = 0
        for n in chunks:
            c.append(*_tokens(1, Bsz, Hkv, n, d, dtype, step))
            step += 1
        q = synth.normal((Bsz, Hkv * G, d), "cpu", 1, 300, 99).to(dtype).cuda()
        sm = 1.0 / np.sqrt(d)
        out1, mask1 = c.decode(q, sm, keep)
        torch.cuda.synchronize()
        out1, mask1 = out1.clone(), mask1.clone()

        path = tmp_path / "cache.pt"
        torch.save(c.state_dict(), path)
        sd = torch.load(path, weights_only=True, map_location=where)
        r = B.Cache.from_state_dict(sd, device="cuda")
        assert r.len == c.len == sum(chunks)
        out2, mask2 = r.decode(q, sm, keep)
        out1b, _ = c.decode(q, sm, keep)
        torch.cuda.synchronize()
        assert torch.equal(mask1, mask2)
        assert torch.equal(out1, out2), "restored cache decodes differently"
        assert torch.equal(out1, out1b), "deterministic decode not repeatable"

        # appends continue identically on both (ring slots and evictions of the window included)
        for n in more:
            k, v = _tokens(1, Bsz, Hkv, n, d, dtype, step)
            c.append(k, v)
            r.append(k, v)
            step += 1
            oa, ma = c.decode(q, sm, keep)
            ob, mb = r.decode(q, sm, keep)
            torch.cuda.synchronize()
            assert torch.equal(ma, mb) and torch.equal(oa, ob), f"decode after appending {n}"
        for nm in c.buffers:
            assert torch.equal(c.buffers[nm], r.buffers[nm]), f"buffer {nm} after further appends"
        assert torch.isfinite(out1).all()
        note("  ok")
    finally:
        B.set_deterministic(False)
