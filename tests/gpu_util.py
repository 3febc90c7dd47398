"""Shared helpers of the GPU parity tests: run the HIP path and the CPU oracle on the
same seeded inputs and compare packed bytes (bit-exact) and outputs (tolerance)."""
import sys

import numpy as np
import torch

from bit_kv_cache_kvq_amd import binding as B

TOL = 2e-3  # max |o_gpu - o_ref| per (sequence, head) row, relative to ||o_ref||_2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_geo(oracle_mod, c: B.Cache, units=None):
    g = oracle_mod.Geometry(batch=c.c.batch, n_kv_heads=c.c.n_kv_heads, head_dim=c.c.head_dim,
                            capacity=c.c.capacity, n_sink=c.c.n_sink, k_format=c.c.k_format,
                            k_hadamard=c.c.k_hadamard, k_ch0_bf16=c.c.k_ch0_bf16,
                            v_format=c.c.v_format, v_clip=float(c.c.v_clip), n_recent=c.c.n_recent,
                            rope_bucket=c.c.rope_bucket)
    table = c.buffers["rope_cs"].view(torch.float32).cpu().numpy() if c.c.rope_bucket else None
    signs = c.buffers["v_qjl_signs"].view(torch.int32).cpu().numpy().view(np.uint32) \
        if c.c.v_format == B.V_KQV else None
    return oracle_mod.OracleCache(g, units=units, rope_table=table, qjl_signs=signs)


def gpu_arrays(c: B.Cache, u0=0, u1=None):
    """Host copies of the GPU buffers for units [u0, u1), shaped like the oracle's arrays."""
    U = c.c.batch * c.c.n_kv_heads
    u1 = U if u1 is None else u1
    d, cap, ns = c.c.head_dim, c.c.capacity, c.c.n_sink
    R = d * (2 if c.c.k_format == B.K_ASYM2 else 4) // 32
    v2 = c.c.v_format == B.V_ASYM2_TOKEN
    shapes = {"k_codes": (R, cap), "k_sz": (d // 32, cap), "k_norm": (cap,), "k_ch0": (cap,),
              "v_codes": (cap // 2, d // 8 if v2 else d // 4),
              "v_sz": (d // 32 if c.c.v_format == B.V_ASYM4_G32 else 1, cap),
              "sink_k": (ns, d), "sink_v": (ns, d), "recent_k": (c.c.n_recent, d), "recent_v": (c.c.n_recent, d)}
    dts = {"k_codes": torch.int32, "k_sz": torch.int32, "k_norm": torch.int16, "k_ch0": torch.int16,
           "v_codes": torch.int32, "v_sz": torch.int32, "sink_k": torch.int16, "sink_v": torch.int16,
           "recent_k": torch.int16, "recent_v": torch.int16}
    out = {}
    for name, shp in shapes.items():
        if name not in c.buffers:
            continue
        t = c.buffers[name].view(dts[name]).view(U, *shp)[u0:u1].cpu().numpy()
        out[name] = t.view(np.uint32 if t.dtype == np.int32 else np.uint16)
    return out


def compare_buffers(c: B.Cache, oc, u0=0, u1=None, what=""):
    ga = gpu_arrays(c, u0, u1)
    for name, arr in ga.items():
        ref = getattr(oc, name)
        if name.startswith("sink"):
            ref = ref[:, : arr.shape[1]]
        if not np.array_equal(arr, ref):
            bad = np.argwhere(arr != ref)
            raise AssertionError(f"{what} buffer {name}: {len(bad)} words differ, first at {bad[0].tolist()}: "
                                 f"gpu {arr[tuple(bad[0])]:#x} oracle {ref[tuple(bad[0])]:#x}")


def compare_outputs(out_gpu, out_ref, what=""):
    """out_gpu: [B, Hq, d] torch; out_ref: [U, G, d] numpy fp64 (same order)."""
    og = out_gpu.detach().cpu().double().numpy().reshape(out_ref.shape)
    err = np.abs(og - out_ref).max(-1)
    nrm = np.linalg.norm(out_ref, axis=-1)
    ratio = err / np.maximum(nrm, 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    assert np.all(np.isfinite(og)), f"{what}: non-finite GPU output"
    assert np.all(err <= TOL * nrm), f"{what}: worst max-err/||o|| = {worst:.3e} > {TOL}"
    return worst


def to_f32_np(t):
    return t.detach().float().cpu().numpy()
