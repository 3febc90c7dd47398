// kvq_api.cpp -- the C ABI of libkvq: host-side validation, buffer sizing, split planning
// and kernel launches.  Everything here runs on the host; validation happens before any
// HIP call, so every error path except KVQ_ERR_HIP leaves the cache untouched.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "kvq_internal.h"

using namespace kvq;

namespace {

std::atomic<int> g_split_tiles{0};
std::atomic<int> g_deterministic{0};
std::atomic<void *> g_decode_ev[2] = {{nullptr}, {nullptr}};

int key_bits(int kfmt) { return kfmt == KVQ_K_ASYM2 ? 2 : 4; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

kvq_status check_geometry(const kvq_cache *c)
{
    if (!c)
        return KVQ_ERR_ARG;
    if (c->batch <= 0 || c->n_kv_heads <= 0 || c->capacity <= 0 || c->len < 0)
        return KVQ_ERR_ARG;
    if ((long long)c->batch * c->n_kv_heads > 65535)
        return KVQ_ERR_UNSUPPORTED;
    if (c->head_dim != 64 && c->head_dim != 128)
        return KVQ_ERR_UNSUPPORTED;
    if (c->capacity % kCapacityQuantum != 0)
        return KVQ_ERR_UNSUPPORTED;
    // per-unit slabs are addressed with 32-bit byte offsets (at most 16 words per position)
    // and the decode work split counts tiles of all units in 32 bits
    if (c->capacity > kMaxCapacity ||
        (long long)c->batch * c->n_kv_heads * (c->capacity / kTile) >= (1ll << 31))
        return KVQ_ERR_UNSUPPORTED;
    if (c->n_sink < 0 || c->n_sink > kMaxSink || c->n_sink >= c->capacity)
        return KVQ_ERR_UNSUPPORTED;
    if (c->k_format < KVQ_K_ASYM2 || c->k_format > KVQ_K_LLOYD4)
        return KVQ_ERR_ARG;
    if ((c->k_hadamard != 0 && c->k_hadamard != 1) || (c->k_ch0_bf16 != 0 && c->k_ch0_bf16 != 1))
        return KVQ_ERR_ARG;
    if (c->k_ch0_bf16 && (c->k_hadamard || c->k_format == KVQ_K_LLOYD4))
        return KVQ_ERR_UNSUPPORTED;
    if (c->v_format != KVQ_V_ASYM4_G32 && c->v_format != KVQ_V_ASYM2_TOKEN && c->v_format != KVQ_V_KQV)
        return KVQ_ERR_ARG;
    if (c->v_format == KVQ_V_ASYM2_TOKEN && !(c->v_clip > 0.0f && c->v_clip <= 1.0f))
        return KVQ_ERR_ARG;
    if (c->n_recent < 0 || c->n_recent > kMaxRecent)
        return KVQ_ERR_UNSUPPORTED;
    if (c->rope_bucket < 0)
        return KVQ_ERR_ARG;
    if (c->rope_bucket != 0 && (c->rope_bucket < kTile || c->rope_bucket > kMaxCapacity ||
                                (c->rope_bucket & (c->rope_bucket - 1)) != 0))
        return KVQ_ERR_UNSUPPORTED;
    if (c->len > c->capacity)
        return KVQ_ERR_CAPACITY;
    return KVQ_OK;
}

size_t units_of(const kvq_cache *c) { return (size_t)c->batch * (size_t)c->n_kv_heads; }

// Bucket-relative RoPE: buckets of the capacity (query records per unit; 1 when off), and
// log2 of the bucket width (0 when off).
int rope_buckets(const kvq_cache *c)
{
    return c->rope_bucket > 0 ? (c->capacity + c->rope_bucket - 1) / c->rope_bucket : 1;
}

int rope_log2(const kvq_cache *c)
{
    int lw = 0;
    while (c->rope_bucket > 0 && (1 << lw) < c->rope_bucket)
        lw++;
    return lw;
}

// End of the quantised positions [n_sink, q_end) when len positions are stored: with a
// recent window of W positions, the W most recent ones (>= n_sink) are still in BF16.
int quant_end(const kvq_cache *c, int len)
{
    if (c->n_recent <= 0)
        return len;
    const int e = len - c->n_recent;
    return e > c->n_sink ? e : c->n_sink;
}

size_t buffer_bytes(const kvq_cache *c, int which)
{
    const size_t U = units_of(c), d = (size_t)c->head_dim, cap = (size_t)c->capacity;
    const size_t ns = (size_t)c->n_sink;
    const bool lloyd = c->k_format == KVQ_K_LLOYD4;
    switch (which) {
    case KVQ_BUF_K_CODES: return U * (d * (size_t)key_bits(c->k_format) / 32) * cap * 4;
    case KVQ_BUF_K_SZ: return lloyd ? 0 : U * (d / 32) * cap * 4;
    case KVQ_BUF_K_NORM: return lloyd ? U * cap * 2 : 0;
    case KVQ_BUF_K_CH0: return c->k_ch0_bf16 ? U * cap * 2 : 0;
    case KVQ_BUF_V_CODES: return U * (cap / 2) * (c->v_format == KVQ_V_ASYM2_TOKEN ? d / 8 : d / 4) * 4;
    case KVQ_BUF_V_SZ: return U * (c->v_format == KVQ_V_ASYM4_G32 ? d / 32 : 1) * cap * 4;
    case KVQ_BUF_SINK_K:
    case KVQ_BUF_SINK_V: return U * ns * d * 2;
    case KVQ_BUF_CODEBOOK: return lloyd ? 16 * 4 : 0;
    case KVQ_BUF_THRESHOLDS: return lloyd ? 15 * 4 : 0;
    case KVQ_BUF_RECENT_K:
    case KVQ_BUF_RECENT_V: return U * (size_t)c->n_recent * d * 2;
    case KVQ_BUF_ROPE_CS: return c->rope_bucket > 0 ? (size_t)rope_buckets(c) * (d / 2) * 2 * 4 : 0;
    case KVQ_BUF_V_CODEBOOK: return c->v_format == KVQ_V_KQV ? 8 * 4 : 0;
    case KVQ_BUF_V_THRESHOLDS: return c->v_format == KVQ_V_KQV ? 7 * 4 : 0;
    case KVQ_BUF_V_QJL_SIGNS: return c->v_format == KVQ_V_KQV ? d / 32 * 4 : 0;
    default: return 0;
    }
}

kvq_status check_buffers(const kvq_cache *c)
{
    const void *ptrs[16] = {c->k_codes,  c->k_sz,       c->k_norm,     c->k_ch0,      c->v_codes,
                            c->v_sz,     c->sink_k,     c->sink_v,     c->codebook,   c->thresholds,
                            c->recent_k, c->recent_v,   c->rope_cs,    c->v_codebook, c->v_thresholds,
                            c->v_qjl_signs};
    for (int i = 0; i < 16; i++) {
        if (buffer_bytes(c, i) == 0)
            continue;
        if (!ptrs[i])
            return KVQ_ERR_ARG;
        if (!aligned16(ptrs[i]))
            return KVQ_ERR_ALIGN;
    }
    return KVQ_OK;
}

struct Plan {
    int tiles_per_unit, n_waves;
};

// Work split of one decode call.  Every unit's positions [0, len) are cut into 128-position
// tiles (at least one, so sink-only and empty contexts still produce their output).  The
// grid is n_waves one-wave workgroups, n_waves >= units: wave w serves unit w % units, and
// the waves of one unit share its tiles (static shares, the last quarter of each stripe drawn
// from a counter at run time; see the decode kernel).  n_waves = the
// resident one-wave workgroups of the kernel instantiation (`slots`), so one pass of waves
// covers the device, capped at one wave per tile; kvq_set_split_tiles overrides it with a
// target number of tiles per wave.
Plan plan_splits(const kvq_cache *c, int len, int slots)
{
    Plan pl;
    pl.tiles_per_unit = (len + kTile - 1) / kTile;
    if (pl.tiles_per_unit < 1)
        pl.tiles_per_unit = 1;
    const long long U = units_of(c);
    const long long total = U * pl.tiles_per_unit;
    long long W = slots > 0 ? slots : 1;
    const int tps = g_split_tiles.load();
    if (tps > 0)
        W = (total + tps - 1) / tps;
    if (W > total)
        W = total;
    if (W > kMaxWaves)
        W = kMaxWaves;
    if (W < U)
        W = U; // one wave per unit at least (more units than slots: the dispatcher balances)
    pl.n_waves = (int)W;
    return pl;
}

// Partial-state slots: one per wave when units share waves (n_waves <= both bounds then).
size_t part_slots(const kvq_cache *c)
{
    const long long max_tiles = (long long)units_of(c) * (c->capacity / kTile);
    return (size_t)(max_tiles < kMaxWaves ? max_tiles : kMaxWaves);
}

} // namespace

extern "C" {

const char *kvq_status_string(kvq_status s)
{
    switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "cache capacity exceeded";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case KVQ_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

size_t kvq_buffer_bytes(const kvq_cache *c, int32_t which)
{
    if (check_geometry(c) != KVQ_OK)
        return 0;
    return buffer_bytes(c, which);
}

kvq_status kvq_validate(const kvq_cache *c)
{
    kvq_status st = check_geometry(c);
    if (st != KVQ_OK)
        return st;
    return check_buffers(c);
}

kvq_status kvq_quant_append(kvq_cache *c, const void *k_new, const void *v_new, int32_t dtype,
                            int32_t n_new, void *stream)
{
    kvq_status st = kvq_validate(c);
    if (st != KVQ_OK)
        return st;
    if (n_new < 0 || (dtype != KVQ_F32 && dtype != KVQ_BF16))
        return KVQ_ERR_ARG;
    if (n_new == 0)
        return KVQ_OK;
    if (!k_new || !v_new)
        return KVQ_ERR_ARG;
    if (!aligned16(k_new) || !aligned16(v_new))
        return KVQ_ERR_ALIGN;
    if ((long long)c->len + n_new > c->capacity)
        return KVQ_ERR_CAPACITY;
    AppendParams p;
    p.k_codes = c->k_codes;
    p.k_sz = c->k_sz;
    p.v_codes = c->v_codes;
    p.v_sz = c->v_sz;
    p.k_norm = c->k_norm;
    p.k_ch0 = c->k_ch0;
    p.sink_k = c->sink_k;
    p.sink_v = c->sink_v;
    p.recent_k = c->recent_k;
    p.recent_v = c->recent_v;
    p.thresholds = c->thresholds;
    p.k_new = k_new;
    p.v_new = v_new;
    p.units = (int)units_of(c);
    p.n_new = n_new;
    p.cap = c->capacity;
    p.len = c->len;
    p.n_sink = c->n_sink;
    p.kfmt = c->k_format;
    p.rotate = c->k_hadamard;
    p.ch0 = c->k_ch0_bf16;
    p.vfmt = c->v_format;
    p.vclip = c->v_clip;
    p.in_bf16 = dtype == KVQ_BF16;
    p.n_recent = c->n_recent;
    p.q_end = quant_end(c, c->len + n_new);
    p.evict = 0;
    p.e0 = 0;
    p.rope_cs = c->rope_cs;
    p.rope_lw = rope_log2(c);
    p.v_codebook = c->v_codebook;
    p.v_thresholds = c->v_thresholds;
    p.v_qjl = c->v_qjl_signs;
    // recent window: first quantise the ring positions that leave it (their slots are
    // overwritten by the new positions of the second launch)
    const int q_old = quant_end(c, c->len);
    const int ev_end = p.q_end < c->len ? p.q_end : c->len;
    if (c->n_recent > 0 && ev_end > q_old) {
        AppendParams e = p;
        e.evict = 1;
        e.e0 = q_old;
        e.n_new = ev_end - q_old;
        if (launch_append(c->head_dim, e, (hipStream_t)stream) != hipSuccess)
            return KVQ_ERR_HIP;
    }
    if (launch_append(c->head_dim, p, (hipStream_t)stream) != hipSuccess)
        return KVQ_ERR_HIP;
    c->len += n_new;
    return KVQ_OK;
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace: partial softmax states [slots][G][D + 4] fp32 (m, l, 2 unused, o), the query records,
// the counters (two per wave place, one per unit)
static size_t part_region_bytes(const kvq_cache *c, int G)
{
    return round256(part_slots(c) * (size_t)G * (size_t)(c->head_dim + 4) * sizeof(float));
}

// BF16 chunk states (query prep -> decode): [unit][chunks][G][D + 4] fp32, chunk 0 the sinks,
// then the window's part of each 64-aligned block of positions it touches (at most
// ceil(n_recent / 64) + 1 blocks; none without a window)
static int bf16_chunk_records(const kvq_cache *c) { return 1 + (c->n_recent > 0 ? (c->n_recent + 63) / 64 + 1 : 0); }

static size_t bstate_region_bytes(const kvq_cache *c, int G)
{
    return round256(units_of(c) * (size_t)bf16_chunk_records(c) * (size_t)G * (size_t)(c->head_dim + 4) *
                    sizeof(float));
}

static size_t qrec_region_bytes(const kvq_cache *c, int G)
{
    return round256(units_of(c) * (size_t)rope_buckets(c) *
                    (size_t)decode_qrec_words(c->head_dim, G, c->k_format) * sizeof(uint32_t));
}

size_t kvq_decode_workspace_bytes(const kvq_cache *c, int32_t n_q_heads)
{
    if (check_geometry(c) != KVQ_OK || n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0)
        return 0;
    const size_t U = units_of(c);
    const size_t G = (size_t)(n_q_heads / c->n_kv_heads);
    // counters: two per wave place (a stripe's tiles drawn and members done, at the place of
    // its first member), then one per unit (members or stripes done)
    const size_t places = part_slots(c) > U ? part_slots(c) : U;
    return part_region_bytes(c, (int)G) + qrec_region_bytes(c, (int)G) + bstate_region_bytes(c, (int)G) +
           round256((2 * places + U) * sizeof(uint32_t));
}

int32_t kvq_decode_splits(const kvq_cache *c, int32_t n_q_heads)
{
    if (check_geometry(c) != KVQ_OK || n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0)
        return 0;
    const int G = n_q_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return 0;
    return plan_splits(c, quant_end(c, c->len), decode_slots(c->head_dim, G, c->k_format, c->v_format)).n_waves;
}

// Everything kvq_decode_attn and kvq_decode_attn_noalloc check before the workspace: the
// descriptor, the query, the output and the grouping.  *G receives the GQA group size.
static kvq_status check_decode_args(const kvq_cache *c, const void *q, int32_t q_dtype, int32_t n_q_heads,
                                    float sm_scale, int32_t keep_groups, const float *out, int *G)
{
    kvq_status st = kvq_validate(c);
    if (st != KVQ_OK)
        return st;
    if (!q || !out || (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16))
        return KVQ_ERR_ARG;
    if (n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0)
        return KVQ_ERR_ARG;
    *G = n_q_heads / c->n_kv_heads;
    if (*G != 1 && *G != 2 && *G != 4 && *G != 8)
        return KVQ_ERR_UNSUPPORTED;
    if (keep_groups < 0 || !isfinite(sm_scale))
        return KVQ_ERR_ARG;
    if (!aligned16(q) || !aligned16(out))
        return KVQ_ERR_ALIGN;
    return KVQ_OK;
}

// The workspace regions of one decode call: partial states [part_slots][G][D + 4] fp32, the
// query records, the counters.
struct WsLayout {
    size_t part, qrec, bstate, ctr; // byte offsets
    size_t total;           // bytes
};

// Layout for any len up to the capacity (kvq_decode_workspace_bytes): partial-state slots for
// the most waves a call of this geometry can use.
static WsLayout layout_bound(const kvq_cache *c, int G)
{
    const size_t U = units_of(c);
    const size_t places = part_slots(c) > U ? part_slots(c) : U;
    WsLayout l;
    l.part = 0;
    l.qrec = part_region_bytes(c, G);
    l.bstate = l.qrec + qrec_region_bytes(c, G);
    l.ctr = l.bstate + bstate_region_bytes(c, G);
    l.total = l.ctr + round256((2 * places + U) * sizeof(uint32_t));
    return l;
}

// Layout of one call with n_waves decode waves (the allocation-free entry point): partial
// states for those waves only.
static WsLayout layout_exact(const kvq_cache *c, int G, int n_waves)
{
    const size_t U = units_of(c);
    WsLayout l;
    l.part = 0;
    l.qrec = round256((size_t)n_waves * (size_t)G * (size_t)(c->head_dim + 4) * sizeof(float));
    l.bstate = l.qrec + qrec_region_bytes(c, G);
    l.ctr = l.bstate + bstate_region_bytes(c, G);
    l.total = l.ctr + round256((2 * (size_t)n_waves + U) * sizeof(uint32_t));
    return l;
}

// The launches of one decode call on a workspace laid out as `l` at ws (checked by the caller).
static kvq_status decode_launch(const kvq_cache *c, const void *q, int32_t q_dtype, int G, float sm_scale,
                                int32_t keep_groups, float *out, uint8_t *mask_out, void *ws, const WsLayout &l,
                                const Plan &pl, void *stream)
{
    const size_t U = units_of(c);
    DecodeParams p;
    p.k_codes = c->k_codes;
    p.k_sz = c->k_sz;
    p.v_codes = c->v_codes;
    p.v_sz = c->v_sz;
    p.k_norm = c->k_norm;
    p.k_ch0 = c->k_ch0;
    p.sink_k = c->sink_k;
    p.sink_v = c->sink_v;
    p.recent_k = c->recent_k;
    p.recent_v = c->recent_v;
    p.codebook = c->codebook;
    p.q = q;
    p.out = out;
    p.mask_out = mask_out;
    p.part = reinterpret_cast<float *>(static_cast<char *>(ws) + l.part);
    p.qprep = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + l.qrec);
    p.tile_ctr = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + l.ctr);
    p.n_kv_heads = c->n_kv_heads;
    p.cap = c->capacity;
    p.len = c->len;
    p.n_sink = c->n_sink;
    p.n_recent = c->n_recent;
    p.q_end = quant_end(c, c->len);
    p.rotate = c->k_hadamard;
    p.ch0 = c->k_ch0_bf16;
    p.keep = keep_groups;
    p.q_bf16 = q_dtype == KVQ_BF16;
    p.sm_log2e = sm_scale * 1.4426950408889634f;
    p.n_units = (int)U;
    p.tiles_per_unit = pl.tiles_per_unit;
    p.n_waves = pl.n_waves;
    p.dynamic = !g_deterministic.load();
    p.n_cu = device_cus();
    p.rope_cs = c->rope_cs;
    p.rope_lw = rope_log2(c);
    p.v_codebook = c->v_codebook;
    p.v_qjl = c->v_qjl_signs;
    p.n_rb = rope_buckets(c);
    p.n_qb = c->rope_bucket > 0 && c->len > 0 ? (c->len + c->rope_bucket - 1) / c->rope_bucket : 1;
    // BF16 positions: the sinks (chunk 0), then the recent window [wlo, len) cut at multiples
    // of 64 positions (one chunk per 64-aligned block it touches)
    p.bstate = reinterpret_cast<float *>(static_cast<char *>(ws) + l.bstate);
    p.bch_max = bf16_chunk_records(c);
    {
        const int ns = c->n_sink < c->len ? c->n_sink : c->len;
        const int wlo = p.q_end > ns ? p.q_end : ns;
        p.n_bch = 1 + (c->len > wlo ? (c->len - 1) / 64 - wlo / 64 + 1 : 0);
    }
    hipEvent_t ev[2] = {static_cast<hipEvent_t>(g_decode_ev[0].load()), static_cast<hipEvent_t>(g_decode_ev[1].load())};
    if (!ev[0] || !ev[1])
        ev[0] = ev[1] = nullptr;
    if (launch_decode(c->head_dim, G, c->k_format, c->v_format, (int)U, p, ev, (hipStream_t)stream) != hipSuccess)
        return KVQ_ERR_HIP;
    return KVQ_OK;
}

static Plan plan_of(const kvq_cache *c, int G)
{
    return plan_splits(c, quant_end(c, c->len), decode_slots(c->head_dim, G, c->k_format, c->v_format));
}

kvq_status kvq_decode_attn(const kvq_cache *c, const void *q, int32_t q_dtype, int32_t n_q_heads,
                           float sm_scale, int32_t keep_groups, float *out, uint8_t *mask_out,
                           void *ws, size_t ws_bytes, void *stream)
{
    int G = 0;
    kvq_status st = check_decode_args(c, q, q_dtype, n_q_heads, sm_scale, keep_groups, out, &G);
    if (st != KVQ_OK)
        return st;
    const WsLayout l = layout_bound(c, G);
    if (!ws || ws_bytes < l.total)
        return KVQ_ERR_WORKSPACE;
    if (!aligned16(ws))
        return KVQ_ERR_ALIGN;
    return decode_launch(c, q, q_dtype, G, sm_scale, keep_groups, out, mask_out, ws, l, plan_of(c, G), stream);
}

size_t kvq_decode_noalloc_scratch_bytes(const kvq_cache *c, int32_t n_q_heads)
{
    if (check_geometry(c) != KVQ_OK || n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0)
        return 0;
    const int G = n_q_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return 0;
    return layout_exact(c, G, plan_of(c, G).n_waves).total;
}

kvq_status kvq_decode_attn_noalloc(const kvq_cache *c, const void *q, int32_t q_dtype, int32_t n_q_heads,
                                   float sm_scale, int32_t keep_groups, float *out, uint8_t *mask_out,
                                   void *stream)
{
    int G = 0;
    kvq_status st = check_decode_args(c, q, q_dtype, n_q_heads, sm_scale, keep_groups, out, &G);
    if (st != KVQ_OK)
        return st;
    const Plan pl = plan_of(c, G);
    const WsLayout l = layout_exact(c, G, pl.n_waves);
    if (l.total > (size_t)KVQ_NOALLOC_SCRATCH_BYTES)
        return KVQ_ERR_WORKSPACE;
    void *scratch = nullptr;
    if (noalloc_scratch(&scratch) != hipSuccess || !scratch)
        return KVQ_ERR_HIP;
    return decode_launch(c, q, q_dtype, G, sm_scale, keep_groups, out, mask_out, scratch, l, pl, stream);
}

void kvq_set_split_tiles(int32_t tiles_per_split) { g_split_tiles.store(tiles_per_split > 0 ? tiles_per_split : 0); }

void kvq_set_deterministic(int32_t on) { g_deterministic.store(on ? 1 : 0); }

kvq_status kvq_probe_stream_read(const void *p, size_t bytes, uint32_t *out, int32_t blocks, void *stream)
{
    if (!p || !out || bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65535)
        return KVQ_ERR_ARG;
    if (!aligned16(p) || !aligned16(out))
        return KVQ_ERR_ALIGN;
    return launch_stream_read(p, bytes, out, blocks, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

void kvq_set_decode_events(void *start_event, void *stop_event)
{
    g_decode_ev[0].store(start_event);
    g_decode_ev[1].store(stop_event);
}

// Symmetric Lloyd-Max quantiser for N(0,1), solved for its positive decision boundaries
// b_1 < ... < b_{H-1} (b_0 = 0, b_H = inf, H = 2^(bits-1) cells on each side) by Newton's
// method on the optimality conditions b_i = (c_{i-1} + c_i) / 2, where c_i is the mean of
// N(0,1) on (b_i, b_{i+1}]: c_i = (pdf(b_i) - pdf(b_{i+1})) / (Q(b_i) - Q(b_{i+1})) with Q
// the upper tail.  The Jacobian is tridiagonal, with dc_i/db_i = pdf(b_i) (c_i - b_i) / P_i
// and dc_i/db_{i+1} = pdf(b_{i+1}) (b_{i+1} - c_i) / P_i (P_i the cell's mass).  The start is
// the equal-mass boundaries; a step is halved until the boundaries stay ordered and the
// residual shrinks.  Centroids and their midpoints are then rounded to fp32.
namespace {

double npdf(double x) { return exp(-0.5 * x * x) * 0.39894228040143267794; }
double nupper(double x) { return 0.5 * erfc(x * 0.70710678118654752440); }

// conditional means of the H positive cells for boundaries b[0..H] (b[0] = 0, b[H] = inf)
void cell_means(const double *b, int H, double *c, double *mass)
{
    for (int i = 0; i < H; i++) {
        const bool last = i == H - 1;
        mass[i] = last ? nupper(b[i]) : nupper(b[i]) - nupper(b[i + 1]);
        c[i] = (last ? npdf(b[i]) : npdf(b[i]) - npdf(b[i + 1])) / mass[i];
    }
}

double residual(const double *b, int H, const double *c, double *F)
{
    double worst = 0.0;
    for (int i = 1; i < H; i++) {
        F[i] = b[i] - 0.5 * (c[i - 1] + c[i]);
        worst = fmax(worst, fabs(F[i]));
    }
    return worst;
}

} // namespace

kvq_status kvq_codebook_gaussian(int32_t bits, float *centroids, float *thresholds)
{
    if (bits < 1 || bits > 6 || !centroids || !thresholds)
        return KVQ_ERR_ARG;
    const int L = 1 << bits, H = L / 2;
    double b[33], c[32], mass[32], F[33], nb[33], nc[32], nmass[32], nF[33];
    b[0] = 0.0;
    for (int i = 1; i < H; i++) { // equal-mass start: Q(b_i) = (1 - i / H) / 2, by bisection
        const double target = 0.5 * (1.0 - (double)i / H);
        double lo = 0.0, hi = 12.0;
        for (int k = 0; k < 200; k++) {
            const double mid = 0.5 * (lo + hi);
            (nupper(mid) > target ? lo : hi) = mid;
        }
        b[i] = 0.5 * (lo + hi);
    }
    cell_means(b, H, c, mass);
    double res = residual(b, H, c, F);
    for (int iter = 0; iter < 200 && res > 1e-15; iter++) {
        // tridiagonal Jacobian of F over b_1 .. b_{H-1}: sub (a), diagonal (d), super (u)
        double a[33], d[33], u[33], rhs[33];
        for (int i = 1; i < H; i++) {
            const double dprev_di = npdf(b[i]) * (b[i] - c[i - 1]) / mass[i - 1]; // d c_{i-1} / d b_i
            const double dcur_di = npdf(b[i]) * (c[i] - b[i]) / mass[i];          // d c_i / d b_i
            d[i] = 1.0 - 0.5 * (dprev_di + dcur_di);
            a[i] = i > 1 ? -0.5 * npdf(b[i - 1]) * (c[i - 1] - b[i - 1]) / mass[i - 1] : 0.0;
            u[i] = i + 1 < H ? -0.5 * npdf(b[i + 1]) * (b[i + 1] - c[i]) / mass[i] : 0.0;
            rhs[i] = -F[i];
        }
        for (int i = 2; i < H; i++) { // forward elimination
            const double w = a[i] / d[i - 1];
            d[i] -= w * u[i - 1];
            rhs[i] -= w * rhs[i - 1];
        }
        double step[33];
        for (int i = H - 1; i >= 1; i--)
            step[i] = (rhs[i] - (i + 1 < H ? u[i] * step[i + 1] : 0.0)) / d[i];
        double lam = 1.0;
        for (int tries = 0; tries < 60; tries++, lam *= 0.5) {
            nb[0] = 0.0;
            bool ordered = true;
            for (int i = 1; i < H; i++) {
                nb[i] = b[i] + lam * step[i];
                ordered = ordered && nb[i] > nb[i - 1];
            }
            if (!ordered)
                continue;
            cell_means(nb, H, nc, nmass);
            const double nres = residual(nb, H, nc, nF);
            if (nres < res || tries == 59) {
                for (int i = 0; i < H; i++) {
                    b[i] = nb[i];
                    c[i] = nc[i];
                    mass[i] = nmass[i];
                }
                for (int i = 1; i < H; i++)
                    F[i] = nF[i];
                res = nres;
                break;
            }
        }
    }
    double full[64]; // the whole codebook, ascending
    for (int i = 0; i < H; i++) {
        full[H + i] = c[i];
        full[H - 1 - i] = -c[i];
    }
    for (int i = 0; i < L; i++)
        centroids[i] = (float)full[i];
    for (int i = 0; i + 1 < L; i++) // decision thresholds: the midpoints (in fp64, then rounded)
        thresholds[i] = (float)(0.5 * (full[i] + full[i + 1]));
    return KVQ_OK;
}

} // extern "C"
