"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/kvq.h declares, sizes buffers per the layout, and rejects bad arguments
before anything is launched (so these calls never reach HIP)."""
import ctypes
import os
import re

import numpy as np
import pytest

from bit_kv_cache_kvq_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # aligned, never dereferenced: validation fails or returns before any launch


def _declared():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_\w+)\s*\(", src)))


def test_exports_every_declared_function():
    L = B.lib()
    names = _declared()
    assert set(B.EXPORTS) == set(names)
    for n in names:
        assert hasattr(L, n), n


def _cache(**kw):
    c = dict(batch=2, n_kv_heads=3, head_dim=128, capacity=512, n_sink=0, k_format=0, k_hadamard=0,
             k_ch0_bf16=0, len=0, v_format=0, v_clip=1.0, n_recent=0, rope_bucket=0)
    c.update(kw)
    s = B.KvqCacheC(*[c[k] for k in ("batch", "n_kv_heads", "head_dim", "capacity", "n_sink", "k_format",
                                      "k_hadamard", "k_ch0_bf16", "len")])
    s.v_format, s.v_clip, s.n_recent = c["v_format"], c["v_clip"], c["n_recent"]
    s.rope_bucket = c["rope_bucket"]
    for name in B.BUF_NAMES:
        setattr(s, name, FAKE)
    return s


def test_buffer_bytes_follow_layout():
    L = B.lib()
    U, d, cap = 6, 128, 512
    s = _cache(k_ch0_bf16=1, n_sink=4)
    nb = [L.kvq_buffer_bytes(ctypes.byref(s), i) for i in range(10)]
    assert nb == [U * 8 * cap * 4, U * 4 * cap * 4, 0, U * cap * 2, U * cap // 2 * 32 * 4, U * 4 * cap * 4,
                  U * 4 * d * 2, U * 4 * d * 2, 0, 0]
    s = _cache(k_format=2, k_hadamard=1, head_dim=64)
    nb = [L.kvq_buffer_bytes(ctypes.byref(s), i) for i in range(10)]
    assert nb == [U * 8 * cap * 4, 0, U * cap * 2, 0, U * cap // 2 * 16 * 4, U * 2 * cap * 4, 0, 0, 64, 60]
    assert L.kvq_buffer_bytes(ctypes.byref(_cache(head_dim=96)), 0) == 0
    # per-token INT2 values: d/8 words per pair, one scale/zero row; recent window rings
    s = _cache(v_format=1, v_clip=0.92, n_recent=256)
    nb = [L.kvq_buffer_bytes(ctypes.byref(s), i) for i in range(12)]
    assert nb[4:6] == [U * cap // 2 * 16 * 4, U * cap * 4]
    assert nb[10:] == [U * 256 * d * 2, U * 256 * d * 2]
    assert L.kvq_buffer_bytes(ctypes.byref(_cache()), 10) == 0
    # bucket-relative RoPE: (cos, sin) per anchor and channel pair, ceil(capacity / w) anchors
    assert L.kvq_buffer_bytes(ctypes.byref(_cache(rope_bucket=128)), 12) == 4 * (d // 2) * 2 * 4
    assert L.kvq_buffer_bytes(ctypes.byref(_cache(rope_bucket=2048)), 12) == 1 * (d // 2) * 2 * 4
    assert L.kvq_buffer_bytes(ctypes.byref(_cache()), 12) == 0
    # KQV values: INT4-layout nibbles, one (rho, residual norm) word per token, 8 centroids,
    # 7 thresholds, d/32 sign words
    s = _cache(v_format=2)
    nb = [L.kvq_buffer_bytes(ctypes.byref(s), i) for i in range(16)]
    assert nb[4:6] == [U * cap // 2 * 32 * 4, U * cap * 4] and nb[13:] == [32, 28, 16]
    assert [L.kvq_buffer_bytes(ctypes.byref(_cache()), i) for i in (13, 14, 15)] == [0, 0, 0]


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), B.KVQ_ERR_UNSUPPORTED),
    (dict(capacity=300), B.KVQ_ERR_UNSUPPORTED),
    (dict(n_sink=65), B.KVQ_ERR_UNSUPPORTED),
    (dict(k_format=7), B.KVQ_ERR_ARG),
    (dict(k_hadamard=1, k_ch0_bf16=1), B.KVQ_ERR_UNSUPPORTED),
    (dict(k_format=2, k_ch0_bf16=1), B.KVQ_ERR_UNSUPPORTED),
    (dict(batch=0), B.KVQ_ERR_ARG),
    (dict(len=513), B.KVQ_ERR_CAPACITY),
    (dict(batch=70000), B.KVQ_ERR_UNSUPPORTED),
    (dict(capacity=(1 << 24) + 256), B.KVQ_ERR_UNSUPPORTED),
    (dict(v_format=3), B.KVQ_ERR_ARG),
    (dict(v_format=1, v_clip=0.0), B.KVQ_ERR_ARG),
    (dict(v_format=1, v_clip=1.5), B.KVQ_ERR_ARG),
    (dict(n_recent=-1), B.KVQ_ERR_UNSUPPORTED),
    (dict(n_recent=1025), B.KVQ_ERR_UNSUPPORTED),
    (dict(rope_bucket=-128), B.KVQ_ERR_ARG),
    (dict(rope_bucket=64), B.KVQ_ERR_UNSUPPORTED),
    (dict(rope_bucket=384), B.KVQ_ERR_UNSUPPORTED),
    (dict(rope_bucket=1 << 25), B.KVQ_ERR_UNSUPPORTED),
])
def test_validate_rejects(kw, code):
    assert B.lib().kvq_validate(ctypes.byref(_cache(**kw))) == code


def test_validate_pointers():
    L = B.lib()
    s = _cache()
    assert L.kvq_validate(ctypes.byref(s)) == B.KVQ_OK
    s.v_sz = None
    assert L.kvq_validate(ctypes.byref(s)) == B.KVQ_ERR_ARG
    s = _cache()
    s.k_codes = FAKE + 4
    assert L.kvq_validate(ctypes.byref(s)) == B.KVQ_ERR_ALIGN
    s = _cache(rope_bucket=256)
    assert L.kvq_validate(ctypes.byref(s)) == B.KVQ_OK
    s.rope_cs = None
    assert L.kvq_validate(ctypes.byref(s)) == B.KVQ_ERR_ARG
    s = _cache()
    s.k_norm = None  # unused by asymmetric keys
    s.codebook = None
    assert L.kvq_validate(ctypes.byref(s)) == B.KVQ_OK


def test_append_errors_leave_len():
    L = B.lib()
    s = _cache(len=500)
    P = ctypes.c_void_p
    assert L.kvq_quant_append(ctypes.byref(s), P(FAKE), P(FAKE), 1, 13, None) == B.KVQ_ERR_CAPACITY
    assert L.kvq_quant_append(ctypes.byref(s), P(FAKE), P(FAKE), 5, 1, None) == B.KVQ_ERR_ARG
    assert L.kvq_quant_append(ctypes.byref(s), P(FAKE), P(FAKE), 1, -1, None) == B.KVQ_ERR_ARG
    assert L.kvq_quant_append(ctypes.byref(s), P(FAKE + 2), P(FAKE), 1, 1, None) == B.KVQ_ERR_ALIGN
    assert L.kvq_quant_append(ctypes.byref(s), None, P(FAKE), 1, 1, None) == B.KVQ_ERR_ARG
    assert L.kvq_quant_append(ctypes.byref(s), P(FAKE), P(FAKE), 1, 0, None) == B.KVQ_OK
    assert s.len == 500
    assert L.kvq_quant_append(None, P(FAKE), P(FAKE), 1, 1, None) == B.KVQ_ERR_ARG


def test_decode_errors():
    L = B.lib()
    s = _cache(len=100)
    P = ctypes.c_void_p
    need = L.kvq_decode_workspace_bytes(ctypes.byref(s), 12)
    assert need > 0
    assert L.kvq_decode_workspace_bytes(ctypes.byref(s), 7) == 0

    def call(hq=12, keep=0, ws_bytes=None, q=FAKE, dt=1, sm=0.088, ws=FAKE):
        return L.kvq_decode_attn(ctypes.byref(s), P(q), dt, hq, sm, keep, P(FAKE), None, P(ws),
                                 need if ws_bytes is None else ws_bytes, None)

    assert call(hq=7) == B.KVQ_ERR_ARG
    assert call(hq=3 * 3) == B.KVQ_ERR_UNSUPPORTED  # G = 3
    assert call(keep=-1) == B.KVQ_ERR_ARG
    assert call(ws_bytes=need - 1) == B.KVQ_ERR_WORKSPACE
    assert call(ws=0) == B.KVQ_ERR_WORKSPACE
    assert call(q=FAKE + 8) == B.KVQ_ERR_ALIGN
    assert call(dt=9) == B.KVQ_ERR_ARG
    assert call(sm=float("nan")) == B.KVQ_ERR_ARG
    assert call(q=0) == B.KVQ_ERR_ARG


def test_split_planner_counts():
    L = B.lib()
    s = _cache(batch=64, n_kv_heads=8, capacity=16640, len=16385, n_sink=4)
    n = L.kvq_decode_splits(ctypes.byref(s), 32)
    tiles = 64 * 8 * ((16385 + 127) // 128)  # 128-position tiles of all units
    assert 1 <= n <= min(tiles, 16384)
    # never more waves than tiles: 8 units of one tile each
    s = _cache(batch=1, n_kv_heads=8, capacity=256, len=100)
    assert 1 <= L.kvq_decode_splits(ctypes.byref(s), 32) <= 8
    # the override sets tiles per wave
    B.set_split_tiles(4)
    try:
        s = _cache(batch=2, n_kv_heads=2, capacity=4096, len=4096)  # 4 units x 32 tiles
        assert L.kvq_decode_splits(ctypes.byref(s), 8) == 32
    finally:
        B.set_split_tiles(0)
    s = _cache(batch=1, n_kv_heads=1, capacity=256, len=0)
    assert L.kvq_decode_splits(ctypes.byref(s), 1) == 1


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert B.status_string(st)
    assert B.status_string(99) == "unknown status"


def test_library_codebook_equals_oracle_codebook(oracle_mod):
    """Two independent Lloyd-Max builders (library host code and oracle) agree bit for bit
    after rounding to fp32."""
    c, t = B.codebook_gaussian(4)
    oc, ot = oracle_mod.codebook_f32(16)
    np.testing.assert_array_equal(np.array(c, np.float32), oc)
    np.testing.assert_array_equal(np.array(t, np.float32), ot)


def test_probe_argument_errors():
    L = B.lib()
    # checked on the host before anything is launched (no GPU needed)
    assert L.kvq_probe_stream_read(None, 1024, FAKE, 4, None) == B.KVQ_ERR_ARG
    assert L.kvq_probe_stream_read(FAKE, 1000, FAKE, 4, None) == B.KVQ_ERR_ARG
    assert L.kvq_probe_stream_read(FAKE, 1024, FAKE, 0, None) == B.KVQ_ERR_ARG
    assert L.kvq_probe_stream_read(FAKE + 8, 1024, FAKE, 4, None) == B.KVQ_ERR_ALIGN


def test_noalloc_entry_refuses_workspace_beyond_its_array():
    """kvq_decode_attn_noalloc sizes the call's workspace on the host and refuses it beyond
    KVQ_NOALLOC_SCRATCH_BYTES before any HIP call."""
    L = B.lib()
    s = _cache(batch=512, n_kv_heads=8, capacity=256)
    need = L.kvq_decode_noalloc_scratch_bytes(ctypes.byref(s), 64)
    assert need > 32 << 20
    st = L.kvq_decode_attn_noalloc(ctypes.byref(s), FAKE, B.KVQ_BF16, 64, 0.088, 0, FAKE, None, None)
    assert st == B.KVQ_ERR_WORKSPACE
    assert L.kvq_decode_attn_noalloc(ctypes.byref(s), None, B.KVQ_BF16, 64, 0.088, 0, FAKE, None, None) == B.KVQ_ERR_ARG
    assert L.kvq_decode_noalloc_scratch_bytes(ctypes.byref(_cache(head_dim=96)), 4) == 0


def test_binding_refuses_other_dtypes_and_devices():
    import torch

    c = B.Cache(1, 1, 64, 256, device="cpu")
    k = torch.zeros(1, 1, 2, 64, dtype=torch.float16)
    with pytest.raises(TypeError):
        c.append(k, k)
    with pytest.raises(TypeError):
        c.decode(torch.zeros(1, 2, 64, dtype=torch.float64), 0.1)
    with pytest.raises(ValueError):
        c.append(torch.zeros(1, 1, 2, 64, device="meta"), torch.zeros(1, 1, 2, 64, device="meta"))


def test_state_dict_round_trip_host():
    """Cache.state_dict() goes through torch.save / torch.load(weights_only=True) and
    from_state_dict() rebuilds a cache with the same geometry, len and bytes (host tensors:
    the descriptor logic only); mismatched states are refused."""
    import io

    import torch

    rng = np.random.default_rng(5)
    c = B.Cache(2, 2, 128, 512, n_sink=4, k_format=B.K_LLOYD4, k_hadamard=1, v_format=B.V_KQV, n_recent=64,
                rope_bucket=128, rope_table=rng.random((4, 64, 2), dtype=np.float32),
                qjl_signs=rng.integers(0, 2**32, 4, dtype=np.uint32), device="cpu")
    for t in c.buffers.values():
        t.copy_(torch.from_numpy(rng.integers(0, 256, t.numel(), dtype=np.uint8)))
    c.c.len = 300
    f = io.BytesIO()
    torch.save(c.state_dict(), f)
    f.seek(0)
    sd = torch.load(f, weights_only=True)
    r = B.Cache.from_state_dict(sd, device="cpu")
    assert r.len == 300 and set(r.buffers) == set(c.buffers)
    for n in B.Cache.GEOMETRY:
        assert getattr(r.c, n) == getattr(c.c, n), n
    for k in c.buffers:
        assert torch.equal(r.buffers[k], c.buffers[k]), k
    bad = dict(sd, len=513)
    with pytest.raises(ValueError):
        B.Cache.from_state_dict(bad, device="cpu")
    short = dict(sd, buffers=dict(sd["buffers"], k_codes=sd["buffers"]["k_codes"][:-16]))
    with pytest.raises(ValueError):
        B.Cache.from_state_dict(short, device="cpu")
    extra = dict(sd, buffers=dict(sd["buffers"], k_ch0=torch.zeros(1024, dtype=torch.uint8)))
    with pytest.raises(ValueError):
        B.Cache.from_state_dict(extra, device="cpu")
