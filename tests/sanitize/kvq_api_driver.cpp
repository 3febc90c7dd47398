// kvq_api_driver.cpp -- the host half of libkvq (kvq_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU.
//
// The launchers, occupancy queries and the allocation-free array that the kernels' sources
// provide are replaced here by host stand-ins.  Every "device" buffer is host memory of
// exactly the size the library asks for (kvq_buffer_bytes, kvq_decode_workspace_bytes,
// kvq_decode_noalloc_scratch_bytes), and the stand-ins write every byte the kernels may
// write and read every byte they may read, so a sizing or layout slip becomes a sanitizer
// report.  The append stand-in also keeps the place of every position of a sequence (sink,
// ring slot of the recent window, quantised) and checks the library's launch plan against
// the packed layout that kvq.h states: each position >= n_sink is quantised exactly once,
// from its ring slot only while that slot still holds it, and after every append the
// positions [n_sink, len - n_recent) are quantised and the rest of [n_sink, len) sit in
// their ring slots.
//
// Prints "kvq_api_driver ok" and exits 0 when every check passes; any failed check exits 1.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "kvq_internal.h"

#define CHECK(cond)                                                                                  \
    do {                                                                                             \
        if (!(cond)) {                                                                               \
            fprintf(stderr, "check failed at %s:%d: %s\n", __FILE__, __LINE__, #cond);               \
            exit(1);                                                                                 \
        }                                                                                            \
    } while (0)

namespace {

// ---- host stand-ins for device memory

void *dev_alloc(size_t bytes)
{
    void *p = nullptr;
    CHECK(posix_memalign(&p, 256, bytes ? bytes : 1) == 0);
    memset(p, 0, bytes ? bytes : 1);
    return p;
}

void touch(void *p, size_t bytes) { memset(p, 0x5a, bytes); }

volatile uint32_t g_sink;
void read_all(const void *p, size_t bytes)
{
    const unsigned char *b = static_cast<const unsigned char *>(p);
    uint32_t x = 0;
    for (size_t i = 0; i < bytes; i++)
        x = x * 31u + b[i];
    g_sink = x;
}

// ---- what the stand-ins know about the call in flight

enum Place { EMPTY = 0, SINK = 1, RING = 2, QUANT = 3 };

struct Sim {
    int n_sink = 0, W = 0, cap = 0, units = 0, D = 0, kfmt = 0, vfmt = 0;
    std::vector<int> place; // per position, same for every unit
    std::vector<int> ring;  // position held by each ring slot (-1: none)
    int appends = 0, evictions = 0;
};

Sim g_sim;
int g_slots = 768;                       // resident decode workgroups reported by decode_slots
const void *g_ws = nullptr;              // workspace of the decode call in flight
size_t g_ws_bytes = 0;
int g_decodes = 0;
int g_expect_G = 0;
void *g_noalloc = nullptr;               // the allocation-free array's stand-in
const kvq_cache *g_cache = nullptr;      // descriptor of the call in flight

int quant_end_of(int len)
{
    if (g_sim.W <= 0)
        return len;
    const int e = len - g_sim.W;
    return e > g_sim.n_sink ? e : g_sim.n_sink;
}

int key_rows(int D, int kfmt) { return D * (kfmt == KVQ_K_ASYM2 ? 2 : 4) / 32; }

// Writes of the encoder for position t of every unit (layout of kvq.h).
void write_quantised(const kvq::AppendParams &p, int D, int t)
{
    const size_t cap = (size_t)p.cap;
    const int R = key_rows(D, p.kfmt);
    for (int u = 0; u < p.units; u++) {
        for (int r = 0; r < R; r++)
            p.k_codes[((size_t)u * R + r) * cap + t] = 0x11111111u;
        if (p.kfmt == KVQ_K_LLOYD4) {
            p.k_norm[(size_t)u * cap + t] = 0x3c00;
        } else {
            for (int g = 0; g < D / 32; g++)
                p.k_sz[((size_t)u * (D / 32) + g) * cap + t] = 0x3c003c00u;
        }
        if (p.ch0)
            p.k_ch0[(size_t)u * cap + t] = 0x3f80;
        const int VW = p.vfmt == KVQ_V_ASYM2_TOKEN ? D / 8 : D / 4;
        uint16_t *vc = reinterpret_cast<uint16_t *>(p.v_codes);
        for (int j = 0; j < VW; j++)
            vc[(((size_t)u * (cap / 2) + t / 2) * VW + j) * 2 + (t & 1)] = 0x1234;
        const int VS = p.vfmt == KVQ_V_ASYM4_G32 ? D / 32 : 1;
        for (int g = 0; g < VS; g++)
            p.v_sz[((size_t)u * VS + g) * cap + t] = 0x3c003c00u;
    }
    if (p.kfmt == KVQ_K_LLOYD4)
        read_all(p.thresholds, 15 * sizeof(float));
    if (p.vfmt == KVQ_V_KQV) {
        read_all(p.v_codebook, 8 * sizeof(float));
        read_all(p.v_thresholds, 7 * sizeof(float));
        read_all(p.v_qjl, (size_t)D / 32 * sizeof(uint32_t));
    }
    if (p.rope_lw)
        read_all(p.rope_cs + (size_t)(t >> p.rope_lw) * D, (size_t)D * sizeof(float));
}

void ring_rows(const kvq::AppendParams &p, int D, int t, bool write)
{
    const size_t W = (size_t)p.n_recent;
    for (int u = 0; u < p.units; u++) {
        const size_t ro = ((size_t)u * W + (size_t)t % W) * D;
        if (write) {
            touch(p.recent_k + ro, (size_t)D * 2);
            touch(p.recent_v + ro, (size_t)D * 2);
        } else {
            read_all(p.recent_k + ro, (size_t)D * 2);
            read_all(p.recent_v + ro, (size_t)D * 2);
        }
    }
}

bool in_ws(const void *p, size_t bytes)
{
    const char *b = static_cast<const char *>(g_ws), *q = static_cast<const char *>(p);
    return q >= b && q + bytes <= b + g_ws_bytes && ((uintptr_t)q & 15u) == 0;
}

bool disjoint(const void *a, size_t na, const void *b, size_t nb)
{
    const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
    return na == 0 || nb == 0 || x + na <= y || y + nb <= x;
}

} // namespace

namespace kvq {

hipError_t launch_append(int D, const AppendParams &p, hipStream_t)
{
    Sim &s = g_sim;
    CHECK(D == s.D && p.units == s.units && p.cap == s.cap && p.n_sink == s.n_sink && p.n_recent == s.W);
    CHECK(p.n_new >= 1);
    CHECK(p.kfmt == s.kfmt && p.vfmt == s.vfmt);
    if (p.evict) {
        CHECK(s.W > 0 && p.e0 >= s.n_sink && p.e0 + p.n_new <= p.len);
        for (int i = 0; i < p.n_new; i++) {
            const int t = p.e0 + i;
            CHECK(s.place[t] == RING && s.ring[t % s.W] == t);
            ring_rows(p, D, t, false);
            write_quantised(p, D, t);
            s.place[t] = QUANT;
        }
        s.evictions++;
        return hipSuccess;
    }
    CHECK(p.len >= 0 && (long long)p.len + p.n_new <= p.cap);
    CHECK(p.q_end == quant_end_of(p.len + p.n_new));
    const size_t elt = p.in_bf16 ? 2 : 4;
    read_all(p.k_new, (size_t)p.units * p.n_new * D * elt);
    read_all(p.v_new, (size_t)p.units * p.n_new * D * elt);
    for (int i = 0; i < p.n_new; i++) {
        const int t = p.len + i;
        CHECK(s.place[t] == EMPTY);
        if (t < p.n_sink) {
            for (int u = 0; u < p.units; u++) {
                touch(p.sink_k + ((size_t)u * p.n_sink + t) * D, (size_t)D * 2);
                touch(p.sink_v + ((size_t)u * p.n_sink + t) * D, (size_t)D * 2);
            }
            s.place[t] = SINK;
        } else if (s.W > 0 && t >= p.q_end) {
            const int prev = s.ring[t % s.W];
            CHECK(prev < 0 || s.place[prev] == QUANT); // its slot's old position left the window
            ring_rows(p, D, t, true);
            s.ring[t % s.W] = t;
            s.place[t] = RING;
        } else {
            write_quantised(p, D, t);
            s.place[t] = QUANT;
        }
    }
    s.appends++;
    return hipSuccess;
}

hipError_t launch_decode(int D, int G, int kfmt, int vfmt, int units, const DecodeParams &p,
                         hipEvent_t const ev[2], hipStream_t)
{
    const kvq_cache *c = g_cache;
    CHECK(c && D == c->head_dim && kfmt == c->k_format && vfmt == c->v_format);
    CHECK(G == g_expect_G && units == c->batch * c->n_kv_heads && p.n_units == units);
    CHECK((ev[0] == nullptr) == (ev[1] == nullptr));
    CHECK(p.len == c->len && p.cap == c->capacity && p.q_end == quant_end_of(c->len));
    // the split: at least one wave per unit, one per tile of the quantised positions at most
    // (unless units outnumber tiles), tiles counted over [0, q_end)
    const int tiles = p.q_end > 0 ? (p.q_end + kTile - 1) / kTile : 1;
    CHECK(p.tiles_per_unit == (tiles > 1 ? tiles : 1));
    CHECK(p.n_waves >= units);
    CHECK(p.n_waves == units || (p.n_waves <= kMaxWaves && p.n_waves <= units * p.tiles_per_unit));
    CHECK(p.n_cu == 256);
    // BF16 chunks: the sinks, then one per 64-aligned block of positions the window
    // [wlo, len) touches
    const int ns = c->n_sink < c->len ? c->n_sink : c->len;
    const int wlo = p.q_end > ns ? p.q_end : ns;
    int blocks = 0;
    for (int a = wlo / 64 * 64; wlo < c->len && a < c->len; a += 64)
        blocks++;
    CHECK(p.n_bch == 1 + blocks);
    CHECK(p.n_bch <= p.bch_max && p.bch_max <= 2 + (c->n_recent + 63) / 64);
    const int n_rb = c->rope_bucket > 0 ? (c->capacity + c->rope_bucket - 1) / c->rope_bucket : 1;
    CHECK(p.n_rb == n_rb && p.n_qb >= 1 && p.n_qb <= n_rb);
    // workspace regions: inside the workspace, 16-byte aligned, pairwise disjoint; then
    // written whole, as the kernels may
    const size_t rec = (size_t)G * (D + 4) * sizeof(float);
    const size_t part_b = p.n_waves > units ? (size_t)p.n_waves * rec : 0;
    const size_t qrec_b = (size_t)units * n_rb * decode_qrec_words(D, G, kfmt) * sizeof(uint32_t);
    const size_t bst_b = (size_t)units * p.bch_max * rec;
    const size_t ctr_b = (2 * (size_t)p.n_waves + units) * sizeof(uint32_t);
    CHECK(in_ws(p.part, part_b) && in_ws(p.qprep, qrec_b) && in_ws(p.bstate, bst_b) && in_ws(p.tile_ctr, ctr_b));
    CHECK(disjoint(p.part, part_b, p.qprep, qrec_b) && disjoint(p.part, part_b, p.bstate, bst_b) &&
          disjoint(p.part, part_b, p.tile_ctr, ctr_b) && disjoint(p.qprep, qrec_b, p.bstate, bst_b) &&
          disjoint(p.qprep, qrec_b, p.tile_ctr, ctr_b) && disjoint(p.bstate, bst_b, p.tile_ctr, ctr_b));
    touch(p.part, part_b);
    touch(p.qprep, qrec_b);
    touch(p.bstate, bst_b);
    touch(p.tile_ctr, ctr_b);
    // query, output, masks
    read_all(p.q, (size_t)units * G * D * (p.q_bf16 ? 2 : 4));
    touch(p.out, (size_t)units * G * D * sizeof(float));
    if (p.mask_out)
        touch(p.mask_out, (size_t)units * n_rb);
    if (kfmt == KVQ_K_LLOYD4)
        read_all(p.codebook, 16 * sizeof(float));
    if (p.rope_lw)
        read_all(p.rope_cs, (size_t)p.n_qb * D * sizeof(float));
    g_decodes++;
    return hipSuccess;
}

hipError_t launch_stream_read(const void *p, size_t bytes, uint32_t *out, int blocks, hipStream_t)
{
    read_all(p, bytes);
    touch(out, (size_t)blocks * sizeof(uint32_t));
    return hipSuccess;
}

// Words of one query record: the kernels' record layout is not under test here, so any
// positive multiple of 64 words of about their size serves.
int decode_qrec_words(int D, int G, int) { return (4 + 4 * D * G / 16 * 8 + 63) / 64 * 64; }

int decode_slots(int, int, int, int) { return g_slots; }

int device_cus() { return 256; }

hipError_t noalloc_scratch(void **ptr)
{
    if (!g_noalloc)
        g_noalloc = dev_alloc(KVQ_NOALLOC_SCRATCH_BYTES);
    *ptr = g_noalloc;
    return hipSuccess;
}

} // namespace kvq

namespace {

// ---- descriptors

struct Bufs {
    std::vector<void *> ptr;
    ~Bufs()
    {
        for (void *p : ptr)
            free(p);
    }
};

// Allocates every buffer the geometry uses at exactly kvq_buffer_bytes and fills the small
// tables (codebooks, thresholds, signs, RoPE) with legal values.
void attach(kvq_cache *c, Bufs &b)
{
    void **slots[16] = {(void **)&c->k_codes,  (void **)&c->k_sz,        (void **)&c->k_norm,
                        (void **)&c->k_ch0,    (void **)&c->v_codes,     (void **)&c->v_sz,
                        (void **)&c->sink_k,   (void **)&c->sink_v,      (void **)&c->codebook,
                        (void **)&c->thresholds, (void **)&c->recent_k,  (void **)&c->recent_v,
                        (void **)&c->rope_cs,  (void **)&c->v_codebook, (void **)&c->v_thresholds,
                        (void **)&c->v_qjl_signs};
    for (int i = 0; i < 16; i++) {
        const size_t n = kvq_buffer_bytes(c, i);
        *slots[i] = nullptr;
        if (n) {
            *slots[i] = dev_alloc(n);
            b.ptr.push_back(*slots[i]);
        }
    }
}

kvq_cache base_cache()
{
    kvq_cache c;
    memset(&c, 0, sizeof(c));
    c.batch = 2;
    c.n_kv_heads = 2;
    c.head_dim = 128;
    c.capacity = 512;
    c.n_sink = 4;
    c.k_format = KVQ_K_ASYM2;
    c.v_format = KVQ_V_ASYM4_G32;
    c.v_clip = 0.92f;
    return c;
}

// Fake, aligned, never dereferenced pointers for the calls that must fail before any launch.
void fake_pointers(kvq_cache *c)
{
    uintptr_t a = 0x10000;
    c->k_codes = (uint32_t *)(a += 256);
    c->k_sz = (uint32_t *)(a += 256);
    c->k_norm = (uint16_t *)(a += 256);
    c->k_ch0 = (uint16_t *)(a += 256);
    c->v_codes = (uint32_t *)(a += 256);
    c->v_sz = (uint32_t *)(a += 256);
    c->sink_k = (uint16_t *)(a += 256);
    c->sink_v = (uint16_t *)(a += 256);
    c->codebook = (const float *)(a += 256);
    c->thresholds = (const float *)(a += 256);
    c->recent_k = (uint16_t *)(a += 256);
    c->recent_v = (uint16_t *)(a += 256);
    c->rope_cs = (const float *)(a += 256);
    c->v_codebook = (const float *)(a += 256);
    c->v_thresholds = (const float *)(a += 256);
    c->v_qjl_signs = (const uint32_t *)(a += 256);
}

uint64_t rng_state = 0x9e3779b97f4a7c15ull;
uint32_t rnd()
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 11);
}

// ---- checks

void check_status_strings()
{
    const int codes[] = {KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_CAPACITY, KVQ_ERR_WORKSPACE,
                         KVQ_ERR_ALIGN, KVQ_ERR_HIP, 7, -99};
    for (int s : codes) {
        const char *m = kvq_status_string((kvq_status)s);
        CHECK(m && strlen(m) > 0);
    }
}

void check_codebook()
{
    for (int bits = 1; bits <= 6; bits++) {
        const int L = 1 << bits;
        float *cent = (float *)malloc(sizeof(float) * L);
        float *thr = (float *)malloc(sizeof(float) * (L - 1));
        CHECK(kvq_codebook_gaussian(bits, cent, thr) == KVQ_OK);
        for (int i = 0; i < L; i++) {
            CHECK(isfinite(cent[i]) && cent[i] == -cent[L - 1 - i]);
            if (i)
                CHECK(cent[i] > cent[i - 1]);
        }
        for (int i = 0; i + 1 < L; i++)
            CHECK(thr[i] > cent[i] && thr[i] < cent[i + 1]);
        free(cent);
        free(thr);
    }
    float cent[64], thr[63];
    CHECK(kvq_codebook_gaussian(0, cent, thr) == KVQ_ERR_ARG);
    CHECK(kvq_codebook_gaussian(7, cent, thr) == KVQ_ERR_ARG);
    CHECK(kvq_codebook_gaussian(4, nullptr, thr) == KVQ_ERR_ARG);
    CHECK(kvq_codebook_gaussian(4, cent, nullptr) == KVQ_ERR_ARG);
}

// buffer sizes against the packed layout of kvq.h, at small and at the largest geometries
void check_buffer_bytes()
{
    const int caps[] = {256, 4096, 1 << 24};
    const int units[][2] = {{1, 1}, {3, 5}, {16383, 1}, {1, 8191}};
    for (int kf = 0; kf < 3; kf++)
        for (int vf = 0; vf < 3; vf++)
            for (int D : {64, 128})
                for (int cap : caps)
                    for (auto &bu : units)
                        for (int W : {0, 256, 1024})
                            for (int rb : {0, 128, 1 << 24}) {
                                kvq_cache c = base_cache();
                                c.batch = bu[0];
                                c.n_kv_heads = bu[1];
                                c.head_dim = D;
                                c.capacity = cap;
                                c.k_format = kf;
                                c.v_format = vf;
                                c.n_recent = W;
                                c.rope_bucket = rb;
                                c.k_ch0_bf16 = kf != KVQ_K_LLOYD4;
                                const uint64_t U = (uint64_t)bu[0] * bu[1];
                                const bool ok = U * (uint64_t)(cap / 128) < (1ull << 31);
                                if (!ok) {
                                    CHECK(kvq_buffer_bytes(&c, KVQ_BUF_K_CODES) == 0);
                                    CHECK(kvq_decode_workspace_bytes(&c, bu[1]) == 0);
                                    continue;
                                }
                                const uint64_t d = D, C = cap, R = d * (kf == KVQ_K_ASYM2 ? 2 : 4) / 32;
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_K_CODES) == U * R * C * 4);
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_K_SZ) == (kf == KVQ_K_LLOYD4 ? 0 : U * (d / 32) * C * 4));
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_K_NORM) == (kf == KVQ_K_LLOYD4 ? U * C * 2 : 0));
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_K_CH0) == (kf == KVQ_K_LLOYD4 ? 0 : U * C * 2));
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_V_CODES) ==
                                      U * (C / 2) * (vf == KVQ_V_ASYM2_TOKEN ? d / 8 : d / 4) * 4);
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_V_SZ) == U * (vf == KVQ_V_ASYM4_G32 ? d / 32 : 1) * C * 4);
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_SINK_K) == U * 4 * d * 2);
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_RECENT_V) == U * (uint64_t)W * d * 2);
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_ROPE_CS) ==
                                      (rb ? (C + rb - 1) / rb * (d / 2) * 2 * 4 : 0));
                                CHECK(kvq_buffer_bytes(&c, KVQ_BUF_V_QJL_SIGNS) == (vf == KVQ_V_KQV ? d / 32 * 4 : 0));
                                CHECK(kvq_buffer_bytes(&c, 16) == 0 && kvq_buffer_bytes(&c, -1) == 0);
                                for (int G : {1, 8}) {
                                    const size_t ws = kvq_decode_workspace_bytes(&c, bu[1] * G);
                                    CHECK(ws > 0 && ws % 256 == 0);
                                }
                            }
}

void check_validation()
{
    struct Case {
        void (*mut)(kvq_cache *);
        kvq_status want;
    };
    const Case cases[] = {
        {[](kvq_cache *c) {}, KVQ_OK},
        {[](kvq_cache *c) { c->batch = 0; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->n_kv_heads = -3; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->batch = 0x7fffffff; c->n_kv_heads = 0x7fffffff; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->batch = 65536; c->n_kv_heads = 1; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->head_dim = 96; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->capacity = 300; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->capacity = 0x7fffff00; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->capacity = (1 << 24) + 256; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->capacity = 1 << 24; c->batch = 16384; c->n_kv_heads = 1; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->capacity = -256; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->len = -1; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->len = c->capacity + 1; }, KVQ_ERR_CAPACITY},
        {[](kvq_cache *c) { c->n_sink = 65; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->n_sink = -1; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->k_format = 3; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->k_format = -1; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->k_hadamard = 2; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->k_ch0_bf16 = 1; c->k_hadamard = 1; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->k_ch0_bf16 = 1; c->k_format = KVQ_K_LLOYD4; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->v_format = 3; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->v_format = KVQ_V_ASYM2_TOKEN; c->v_clip = 0.0f; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->v_format = KVQ_V_ASYM2_TOKEN; c->v_clip = NAN; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->v_format = KVQ_V_ASYM2_TOKEN; c->v_clip = 1.5f; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->n_recent = 1025; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->n_recent = -1; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->rope_bucket = -128; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->rope_bucket = (int)0x80000000u; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->rope_bucket = 64; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->rope_bucket = 384; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->rope_bucket = 1 << 30; }, KVQ_ERR_UNSUPPORTED},
        {[](kvq_cache *c) { c->k_codes = nullptr; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->v_sz = (uint32_t *)((char *)c->v_sz + 4); }, KVQ_ERR_ALIGN},
        {[](kvq_cache *c) { c->rope_bucket = 128; c->rope_cs = nullptr; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->v_format = KVQ_V_KQV; c->v_qjl_signs = nullptr; }, KVQ_ERR_ARG},
        {[](kvq_cache *c) { c->k_format = KVQ_K_LLOYD4; c->codebook = (const float *)((char *)c->codebook + 8); }, KVQ_ERR_ALIGN},
        {[](kvq_cache *c) { c->n_recent = 64; c->recent_v = nullptr; }, KVQ_ERR_ARG},
    };
    for (const Case &k : cases) {
        kvq_cache c = base_cache();
        fake_pointers(&c);
        k.mut(&c);
        CHECK(kvq_validate(&c) == k.want);
        // every entry point refuses an invalid descriptor with the same code, launching nothing
        const int before = g_decodes;
        if (k.want != KVQ_OK) {
            CHECK(kvq_quant_append(&c, (void *)0x1000, (void *)0x2000, KVQ_F32, 1, nullptr) == k.want);
            CHECK(kvq_decode_attn(&c, (void *)0x1000, KVQ_F32, c.n_kv_heads, 0.1f, 0, (float *)0x2000, nullptr,
                                  (void *)0x3000, (size_t)1 << 40, nullptr) == k.want);
            CHECK(kvq_decode_attn_noalloc(&c, (void *)0x1000, KVQ_F32, c.n_kv_heads, 0.1f, 0, (float *)0x2000,
                                          nullptr, nullptr) == k.want);
            CHECK(g_decodes == before);
        }
    }
    CHECK(kvq_validate(nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_buffer_bytes(nullptr, 0) == 0);
    CHECK(kvq_decode_workspace_bytes(nullptr, 1) == 0);
    CHECK(kvq_decode_noalloc_scratch_bytes(nullptr, 1) == 0);
    CHECK(kvq_decode_splits(nullptr, 1) == 0);
}

void check_probe()
{
    uint32_t *buf = (uint32_t *)dev_alloc(4096), *out = (uint32_t *)dev_alloc(64 * 4);
    CHECK(kvq_probe_stream_read(buf, 4096, out, 64, nullptr) == KVQ_OK);
    CHECK(kvq_probe_stream_read(buf, 0, out, 64, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_probe_stream_read(buf, 4095, out, 64, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_probe_stream_read(buf, 4096, out, 0, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_probe_stream_read(buf, 4096, out, 65536, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_probe_stream_read(nullptr, 4096, out, 1, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_probe_stream_read((char *)buf + 4, 4080, out, 1, nullptr) == KVQ_ERR_ALIGN);
    free(buf);
    free(out);
}

// The place of every position after an append (same for all units).
void check_places(const kvq_cache &c)
{
    const int qe = quant_end_of(c.len);
    for (int t = 0; t < c.capacity; t++) {
        const int pl = g_sim.place[t];
        if (t >= c.len)
            CHECK(pl == EMPTY);
        else if (t < c.n_sink)
            CHECK(pl == SINK);
        else if (t < qe)
            CHECK(pl == QUANT);
        else
            CHECK(pl == RING && g_sim.ring[t % g_sim.W] == t);
    }
}

// One decode through each entry point on an exact-size workspace, with masks and events.
void decode_both(kvq_cache &c, int G, int dtype, void *q, float *out, uint8_t *mask)
{
    g_cache = &c;
    g_expect_G = G;
    const int nq = c.n_kv_heads * G;
    const size_t ws_bytes = kvq_decode_workspace_bytes(&c, nq);
    CHECK(ws_bytes > 0);
    void *ws = dev_alloc(ws_bytes);
    g_ws = ws;
    g_ws_bytes = ws_bytes;
    const int keep = (int)(rnd() % 9);
    int before = g_decodes;
    CHECK(kvq_decode_attn(&c, q, dtype, nq, 0.0884f, keep, out, mask, ws, ws_bytes, nullptr) == KVQ_OK);
    CHECK(g_decodes == before + 1);
    // the error paths of the workspace and the arguments launch nothing
    before = g_decodes;
    CHECK(kvq_decode_attn(&c, q, dtype, nq, 0.0884f, keep, out, mask, ws, ws_bytes - 1, nullptr) == KVQ_ERR_WORKSPACE);
    CHECK(kvq_decode_attn(&c, q, dtype, nq, 0.0884f, keep, out, mask, nullptr, ws_bytes, nullptr) == KVQ_ERR_WORKSPACE);
    CHECK(kvq_decode_attn(&c, q, dtype, nq, 0.0884f, keep, out, mask, (char *)ws + 8, ws_bytes, nullptr) == KVQ_ERR_ALIGN);
    CHECK(kvq_decode_attn(&c, (char *)q + 4, dtype, nq, 0.0884f, keep, out, mask, ws, ws_bytes, nullptr) == KVQ_ERR_ALIGN);
    CHECK(kvq_decode_attn(&c, q, dtype, nq, NAN, keep, out, mask, ws, ws_bytes, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_decode_attn(&c, q, dtype, nq, INFINITY, keep, out, mask, ws, ws_bytes, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_decode_attn(&c, q, dtype, nq, 0.1f, -1, out, mask, ws, ws_bytes, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_decode_attn(&c, q, 5, nq, 0.1f, 0, out, mask, ws, ws_bytes, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_decode_attn(&c, q, dtype, c.n_kv_heads * 3, 0.1f, 0, out, mask, ws, ws_bytes, nullptr) ==
          KVQ_ERR_UNSUPPORTED);
    if (c.n_kv_heads > 1)
        CHECK(kvq_decode_attn(&c, q, dtype, nq + 1, 0.1f, 0, out, mask, ws, ws_bytes, nullptr) == KVQ_ERR_ARG);
    CHECK(kvq_decode_attn(&c, nullptr, dtype, nq, 0.1f, 0, out, mask, ws, ws_bytes, nullptr) == KVQ_ERR_ARG);
    CHECK(g_decodes == before);
    free(ws);
    // the allocation-free entry point: its regions must fit the bytes it reports for this call
    const size_t nb = kvq_decode_noalloc_scratch_bytes(&c, nq);
    CHECK(nb > 0 && nb <= ws_bytes);
    void *scratch = nullptr;
    CHECK(kvq::noalloc_scratch(&scratch) == hipSuccess);
    g_ws = scratch;
    g_ws_bytes = nb;
    before = g_decodes;
    CHECK(kvq_decode_attn_noalloc(&c, q, dtype, nq, 0.0884f, keep, out, mask, nullptr) == KVQ_OK);
    CHECK(g_decodes == before + 1);
    CHECK(kvq_decode_splits(&c, nq) >= c.batch * c.n_kv_heads);
    g_ws = nullptr;
    g_ws_bytes = 0;
}

// Random appends to the capacity with decodes in between, on exact-size buffers.
void run_sequence(int D, int cap, int n_sink, int W, int kf, int vf, int rb, int batch, int hkv, int G)
{
    kvq_cache c = base_cache();
    c.batch = batch;
    c.n_kv_heads = hkv;
    c.head_dim = D;
    c.capacity = cap;
    c.n_sink = n_sink;
    c.k_format = kf;
    c.v_format = vf;
    c.n_recent = W;
    c.rope_bucket = rb;
    c.k_hadamard = kf == KVQ_K_LLOYD4 ? (int)(rnd() & 1) : 0;
    c.k_ch0_bf16 = kf != KVQ_K_LLOYD4 ? (int)(rnd() & 1) : 0;
    Bufs b;
    attach(&c, b);
    CHECK(kvq_validate(&c) == KVQ_OK);
    g_sim = Sim();
    g_sim.n_sink = n_sink;
    g_sim.W = W;
    g_sim.cap = cap;
    g_sim.units = batch * hkv;
    g_sim.D = D;
    g_sim.kfmt = kf;
    g_sim.vfmt = vf;
    g_sim.place.assign(cap, EMPTY);
    g_sim.ring.assign(W > 0 ? W : 1, -1);
    g_cache = &c;

    const int U = batch * hkv;
    const int dtype = (int)(rnd() & 1);
    const size_t elt = dtype == KVQ_BF16 ? 2 : 4;
    void *q = dev_alloc((size_t)U * G * D * elt);
    float *out = (float *)dev_alloc((size_t)U * G * D * sizeof(float));
    const int n_rb = rb ? (cap + rb - 1) / rb : 1;
    uint8_t *mask = (uint8_t *)dev_alloc((size_t)U * n_rb);
    void *ev[2] = {(void *)0x100, (void *)0x200};

    decode_both(c, G, dtype, q, out, nullptr); // empty cache
    while (c.len < cap) {
        const int room = cap - c.len;
        const uint32_t pick = rnd() % 8;
        int n = pick < 3 ? 1 : pick < 6 ? (int)(rnd() % 80) + 1 : (int)(rnd() % 700) + 1;
        if (n > room)
            n = room;
        void *kn = dev_alloc((size_t)U * n * D * elt), *vn = dev_alloc((size_t)U * n * D * elt);
        const int len0 = c.len;
        // refusals leave the cache as it was
        CHECK(kvq_quant_append(&c, kn, vn, dtype, room + 1, nullptr) == KVQ_ERR_CAPACITY);
        CHECK(kvq_quant_append(&c, kn, vn, dtype, -1, nullptr) == KVQ_ERR_ARG);
        CHECK(kvq_quant_append(&c, kn, vn, 9, n, nullptr) == KVQ_ERR_ARG);
        CHECK(kvq_quant_append(&c, nullptr, vn, dtype, n, nullptr) == KVQ_ERR_ARG);
        CHECK(kvq_quant_append(&c, kn, (char *)vn + 2, dtype, n, nullptr) == KVQ_ERR_ALIGN);
        CHECK(kvq_quant_append(&c, kn, vn, dtype, 0, nullptr) == KVQ_OK);
        CHECK(c.len == len0);
        CHECK(kvq_quant_append(&c, kn, vn, dtype, n, nullptr) == KVQ_OK);
        CHECK(c.len == len0 + n);
        free(kn);
        free(vn);
        check_places(c);
        if (rnd() % 3 == 0) {
            g_slots = (int)(rnd() % 4 == 0 ? 1 : rnd() % 4 == 0 ? 100000 : 768);
            kvq_set_split_tiles((int)(rnd() % 4 == 0 ? rnd() % 5 : 0));
            kvq_set_deterministic((int)(rnd() & 1));
            kvq_set_decode_events(rnd() & 1 ? ev[0] : nullptr, rnd() & 1 ? ev[1] : nullptr);
            decode_both(c, G, dtype, q, out, rnd() & 1 ? mask : nullptr);
        }
    }
    decode_both(c, G, dtype, q, out, mask);
    kvq_set_split_tiles(0);
    kvq_set_deterministic(0);
    kvq_set_decode_events(nullptr, nullptr);
    g_slots = 768;
    free(q);
    free(out);
    free(mask);
}

// The allocation-free entry point refuses a call whose workspace exceeds its array, before
// anything is enqueued.
void check_noalloc_limit()
{
    kvq_cache c = base_cache();
    c.batch = 64;
    c.n_kv_heads = 8;
    c.capacity = 1 << 16;
    c.len = c.capacity;
    c.n_recent = 1024;
    fake_pointers(&c);
    g_cache = &c;
    g_slots = 16384;
    const size_t nb = kvq_decode_noalloc_scratch_bytes(&c, 64);
    CHECK(nb > (size_t)KVQ_NOALLOC_SCRATCH_BYTES);
    const int before = g_decodes;
    CHECK(kvq_decode_attn_noalloc(&c, (void *)0x1000, KVQ_F32, 64, 0.1f, 0, (float *)0x2000, nullptr, nullptr) ==
          KVQ_ERR_WORKSPACE);
    CHECK(g_decodes == before);
    CHECK(kvq_decode_noalloc_scratch_bytes(&c, 3 * 8) == 0); // G = 3
    CHECK(kvq_decode_noalloc_scratch_bytes(&c, 63) == 0);
    g_slots = 768;
}

} // namespace

const int kSinks[4] = {0, 1, 4, 64};
const int kGroups[4] = {1, 2, 4, 8};

int main()
{
    check_status_strings();
    check_codebook();
    check_buffer_bytes();
    check_validation();
    check_probe();
    check_noalloc_limit();
    int runs = 0;
    for (int kf = 0; kf < 3; kf++)
        for (int vf = 0; vf < 3; vf++)
            for (int W : {0, 64, 100, 256}) {
                const int D = (runs & 1) ? 64 : 128;
                const int ns = kSinks[runs % 4];
                const int cap = (runs % 3 == 0) ? 768 : 512;
                const int rb = (runs % 5 == 0) ? 128 : (runs % 5 == 1 ? 256 : 0);
                const int G = kGroups[(runs / 2) % 4];
                run_sequence(D, cap, ns, W, kf, vf, rb, 1 + runs % 3, 1 + (runs / 3) % 2, G);
                runs++;
            }
    run_sequence(128, 256, 64, 1024, KVQ_K_ASYM2, KVQ_V_ASYM2_TOKEN, 0, 2, 2, 4); // window > capacity
    run_sequence(64, 256, 0, 1, KVQ_K_ASYM4, KVQ_V_ASYM4_G32, 0, 1, 1, 1);         // window of one
    printf("kvq_api_driver ok: %d sequences, %d decodes\n", runs + 2, g_decodes);
    free(g_noalloc);
    return 0;
}
