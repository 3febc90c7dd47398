/*
 * oracle_driver.c -- the oracle (oracle/kvq_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer.
 *
 * Every buffer is allocated at exactly the size of the packed layout of its format, and a
 * buffer a format does not use is a zero-byte allocation, so any access outside what the
 * layout gives that format is a sanitizer report.  Inputs span several binades, exact
 * zeros (degenerate groups), ties and inputs near the fp16 limit, so the encoder's casts and
 * shifts are exercised at their ends.  Beyond running clean, each decode is checked against
 * two properties that hold for any correct attention: without pruning every output channel
 * lies between the smallest and the largest decoded value of that channel over the
 * positions, and a cache of length 0 gives zeros.
 *
 * Prints "oracle_driver ok" and exits 0 when every check passes; any failed check exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define CHECK(cond)                                                                          \
    do {                                                                                     \
        if (!(cond)) {                                                                       \
            fprintf(stderr, "check failed at %s:%d: %s\n", __FILE__, __LINE__, #cond);       \
            exit(1);                                                                         \
        }                                                                                    \
    } while (0)

/* the oracle's entry points */
uint16_t oracle_f32_to_f16(float f);
float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float f);
float oracle_bf16_to_f32(uint16_t b);
void oracle_fwht_f32(float *y, int d);
void oracle_fwht_f64(double *y, int d);
float oracle_tree_sum_f32(float *a, int n);
int oracle_lloyd_max_gaussian(int levels, double tol, int max_iter, double *cent, double *thr);
uint32_t oracle_prune_mask(const float *qt, int G, int d, int m);
void oracle_quant_append(int d, int cap, int n_sink, int kfmt, int rotate, int ch0, int vfmt, float vclip,
                         int n_recent, uint32_t *k_codes, uint32_t *k_sz, uint16_t *k_norm, uint16_t *k_ch0,
                         uint32_t *v_codes, uint32_t *v_sz, uint16_t *sink_k, uint16_t *sink_v,
                         uint16_t *recent_k, uint16_t *recent_v, int rope_w, const float *rope_cs,
                         const float *vcent, const float *vthr, const uint32_t *qjl, const float *cent,
                         const float *thr, int n_units, int t0, int n_new, const float *k_new,
                         const float *v_new);
void oracle_dequant_unit(int d, int cap, int n_sink, int kfmt, int rotate, int ch0, int vfmt, float vclip,
                         int n_recent, uint32_t *k_codes, uint32_t *k_sz, uint16_t *k_norm, uint16_t *k_ch0,
                         uint32_t *v_codes, uint32_t *v_sz, uint16_t *sink_k, uint16_t *sink_v,
                         uint16_t *recent_k, uint16_t *recent_v, int rope_w, const float *rope_cs,
                         const float *vcent, const float *vthr, const uint32_t *qjl, const float *cent,
                         int unit, int len, double *kh, double *vh);
void oracle_decode_attn(int d, int cap, int n_sink, int kfmt, int rotate, int ch0, int vfmt, float vclip,
                        int n_recent, uint32_t *k_codes, uint32_t *k_sz, uint16_t *k_norm, uint16_t *k_ch0,
                        uint32_t *v_codes, uint32_t *v_sz, uint16_t *sink_k, uint16_t *sink_v,
                        uint16_t *recent_k, uint16_t *recent_v, int rope_w, const float *rope_cs,
                        const float *vcent, const float *vthr, const uint32_t *qjl, const float *cent,
                        int n_units, int len, int G, const float *q, double sm, int keep_groups, double *out,
                        uint8_t *mask_out, double *logits_out);

enum { K_ASYM2 = 0, K_ASYM4 = 1, K_LLOYD4 = 2, K_ASYM8 = 3 };
enum { V_ASYM4 = 0, V_INT2_TOKEN = 1, V_KQV = 2 };

static uint64_t rng = 0x243f6a8885a308d3ull;
static uint32_t rnd(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 11);
}
static float unif(void) { return (float)((rnd() & 0xFFFFFF) / 16777216.0 * 2.0 - 1.0); }

/* exact-size allocation; zero bytes for a buffer the format does not use */
static void *xalloc(size_t bytes)
{
    void *p = malloc(bytes);
    CHECK(p || bytes == 0);
    if (bytes)
        memset(p, 0, bytes);
    return p;
}

static void check_conversions(void)
{
    for (uint32_t h = 0; h < 65536; h++) {
        const float f = oracle_f16_to_f32((uint16_t)h);
        if (isnan(f))
            continue;
        CHECK(oracle_f32_to_f16(f) == h);
        CHECK(oracle_bf16_to_f32(oracle_f32_to_bf16(f)) == oracle_bf16_to_f32(oracle_f32_to_bf16(f)));
    }
    for (int i = 0; i < 200000; i++) {
        uint32_t x = rnd() ^ (rnd() << 21);
        float f;
        memcpy(&f, &x, 4);
        const uint16_t h = oracle_f32_to_f16(f), b = oracle_f32_to_bf16(f);
        const float fh = oracle_f16_to_f32(h), fb = oracle_bf16_to_f32(b);
        if (isnan(f)) {
            CHECK(isnan(fh) && isnan(fb));
        } else {
            CHECK(fabsf(fh) <= 65504.0f || isinf(fh));
            CHECK(isinf(fb) || fabsf(fb - f) <= fabsf(f) * 0x1p-8f + 0x1p-134f); /* half an ulp */
        }
    }
}

static void check_transforms(void)
{
    for (int d = 64; d <= 128; d *= 2) {
        float *y = xalloc(sizeof(float) * d), *a = xalloc(sizeof(float) * d);
        double *z = xalloc(sizeof(double) * d);
        for (int i = 0; i < d; i++) {
            y[i] = unif();
            z[i] = y[i];
            a[i] = 1.0f;
        }
        oracle_fwht_f32(y, d);
        oracle_fwht_f64(z, d);
        oracle_fwht_f64(z, d); /* H H = d I */
        CHECK(oracle_tree_sum_f32(a, d) == (float)d);
        for (int i = 0; i < d; i++)
            CHECK(isfinite(y[i]) && isfinite(z[i]));
        free(y);
        free(a);
        free(z);
    }
    for (int L = 2; L <= 64; L *= 2) {
        double *cent = xalloc(sizeof(double) * L), *thr = xalloc(sizeof(double) * (L - 1));
        const int it = oracle_lloyd_max_gaussian(L, 1e-12, 100000, cent, thr);
        CHECK(it >= 0);
        for (int i = 0; i + 1 < L; i++)
            CHECK(cent[i] < thr[i] && thr[i] < cent[i + 1]);
        free(cent);
        free(thr);
    }
    for (int d = 64; d <= 128; d *= 2)
        for (int G = 1; G <= 8; G *= 2)
            for (int m = -1; m <= d / 16 + 1; m++) {
                float *qt = xalloc(sizeof(float) * G * d);
                for (int i = 0; i < G * d; i++)
                    qt[i] = (i % 7 == 0) ? 0.0f : unif() * (float)(1 << (i % 5));
                const uint32_t mask = oracle_prune_mask(qt, G, d, m);
                const int kept = __builtin_popcount(mask);
                CHECK(kept == ((m <= 0 || m >= d / 16) ? d / 16 : m));
                free(qt);
            }
}

typedef struct {
    int U, d, cap, n_sink, kfmt, rotate, ch0, vfmt, W, rope_w;
    float vclip;
    uint32_t *k_codes, *k_sz, *v_codes, *v_sz, *qjl;
    uint16_t *k_norm, *k_ch0, *sink_k, *sink_v, *recent_k, *recent_v;
    float *rope_cs, *vcent, *vthr, *cent, *thr;
} cache;

static int key_bits(int kfmt) { return kfmt == K_ASYM2 ? 2 : kfmt == K_ASYM8 ? 8 : 4; }

static void cache_alloc(cache *c)
{
    const size_t U = c->U, d = c->d, cap = c->cap;
    const int lloyd = c->kfmt == K_LLOYD4, kqv = c->vfmt == V_KQV;
    c->k_codes = xalloc(U * (d * key_bits(c->kfmt) / 32) * cap * 4);
    c->k_sz = xalloc(lloyd ? 0 : U * (d / 32) * cap * 4);
    c->k_norm = xalloc(lloyd ? U * cap * 2 : 0);
    c->k_ch0 = xalloc(c->ch0 ? U * cap * 2 : 0);
    c->v_codes = xalloc(U * (cap / 2) * (c->vfmt == V_INT2_TOKEN ? d / 8 : d / 4) * 4);
    c->v_sz = xalloc(U * (c->vfmt == V_ASYM4 ? d / 32 : 1) * cap * 4);
    c->sink_k = xalloc(U * (size_t)c->n_sink * d * 2);
    c->sink_v = xalloc(U * (size_t)c->n_sink * d * 2);
    c->recent_k = xalloc(U * (size_t)c->W * d * 2);
    c->recent_v = xalloc(U * (size_t)c->W * d * 2);
    const size_t nb = c->rope_w ? (cap + c->rope_w - 1) / c->rope_w : 0;
    c->rope_cs = xalloc(nb * (d / 2) * 2 * sizeof(float));
    for (size_t b = 0; b < nb; b++)
        for (size_t i = 0; i < d / 2; i++) {
            const double ang = (double)(b * c->rope_w) * pow(10000.0, -2.0 * (double)i / (double)d);
            c->rope_cs[(b * (d / 2) + i) * 2] = (float)cos(ang);
            c->rope_cs[(b * (d / 2) + i) * 2 + 1] = (float)sin(ang);
        }
    c->qjl = xalloc(kqv ? d / 32 * 4 : 0);
    for (size_t i = 0; kqv && i < d / 32; i++)
        c->qjl[i] = rnd() ^ (rnd() << 16);
    c->vcent = xalloc(kqv ? 8 * sizeof(float) : 0);
    c->vthr = xalloc(kqv ? 7 * sizeof(float) : 0);
    c->cent = xalloc(lloyd ? 16 * sizeof(float) : 0);
    c->thr = xalloc(lloyd ? 15 * sizeof(float) : 0);
    double cb[16], tb[15];
    if (kqv) {
        oracle_lloyd_max_gaussian(8, 1e-13, 200000, cb, tb);
        for (int i = 0; i < 8; i++)
            c->vcent[i] = (float)cb[i];
        for (int i = 0; i < 7; i++)
            c->vthr[i] = (float)tb[i];
    }
    if (lloyd) {
        oracle_lloyd_max_gaussian(16, 1e-13, 200000, cb, tb);
        for (int i = 0; i < 16; i++)
            c->cent[i] = (float)cb[i];
        for (int i = 0; i < 15; i++)
            c->thr[i] = (float)tb[i];
    }
}

static void cache_free(cache *c)
{
    void *p[] = {c->k_codes, c->k_sz, c->k_norm, c->k_ch0, c->v_codes, c->v_sz, c->sink_k, c->sink_v,
                 c->recent_k, c->recent_v, c->rope_cs, c->qjl, c->vcent, c->vthr, c->cent, c->thr};
    for (size_t i = 0; i < sizeof(p) / sizeof(p[0]); i++)
        free(p[i]);
}

/* one token's key and value: several binades, exact zeros, repeated values, and (formats
 * whose parameters are per group or per token) entries near the fp16 limit */
static void fill_token(const cache *c, float *k, float *v)
{
    const int kind = (int)(rnd() % 8);
    const int big_k = c->kfmt != K_LLOYD4, big_v = c->vfmt != V_KQV;
    for (int i = 0; i < c->d; i++) {
        float a = unif(), b = unif();
        switch (kind) {
        case 0: a = b = 0.0f; break;                            /* degenerate groups */
        case 1: a = 0.25f * (float)(i % 3); b = -a; break;      /* ties, repeats */
        case 2: a *= 1e-6f; b *= 1e-6f; break;                  /* fp16 subnormal scales */
        case 3: /* the anchor rotation of RoPE can grow an entry by up to sqrt(2) */
            a *= big_k ? (c->rope_w ? 4.5e4f : 5e4f) : 3e3f;
            b *= big_v ? 5e4f : 2e3f;
            break;
        case 4: a = (i & 1) ? -0.0f : 0.0f; b *= 100.0f; break;
        default: a *= (float)(1 << (i % 6)); b *= 3.0f; break;
        }
        k[i] = a;
        v[i] = b;
    }
}

#define CACHE_ARGS(c)                                                                               \
    (c)->d, (c)->cap, (c)->n_sink, (c)->kfmt, (c)->rotate, (c)->ch0, (c)->vfmt, (c)->vclip, (c)->W,  \
        (c)->k_codes, (c)->k_sz, (c)->k_norm, (c)->k_ch0, (c)->v_codes, (c)->v_sz, (c)->sink_k,     \
        (c)->sink_v, (c)->recent_k, (c)->recent_v, (c)->rope_w, (c)->rope_cs, (c)->vcent, (c)->vthr, \
        (c)->qjl, (c)->cent

static void decode_and_check(const cache *c, int len, int G, int keep)
{
    const int U = c->U, d = c->d;
    const int n_rb = c->rope_w ? (c->cap + c->rope_w - 1) / c->rope_w : 1;
    float *q = xalloc(sizeof(float) * U * G * d);
    for (int i = 0; i < U * G * d; i++)
        q[i] = unif() * (float)(1 + (i % 11 == 0) * 40);
    double *out = xalloc(sizeof(double) * U * G * d);
    double *logits = xalloc(sizeof(double) * U * G * (len > 0 ? len : 0));
    uint8_t *mask = xalloc((size_t)U * n_rb);
    oracle_decode_attn(CACHE_ARGS(c), U, len, G, q, 0.0884, keep, out, mask, len > 0 ? logits : NULL);
    double *kh = xalloc(sizeof(double) * (len > 0 ? len : 0) * d), *vh = xalloc(sizeof(double) * (len > 0 ? len : 0) * d);
    for (int u = 0; u < U; u++) {
        if (len > 0)
            oracle_dequant_unit(CACHE_ARGS(c), u, len, kh, vh);
        for (int h = 0; h < G; h++)
            for (int i = 0; i < d; i++) {
                const double o = out[((size_t)u * G + h) * d + i];
                CHECK(isfinite(o));
                if (len == 0) {
                    CHECK(o == 0.0);
                    continue;
                }
                double lo = INFINITY, hi = -INFINITY;
                for (int t = 0; t < len; t++) {
                    lo = fmin(lo, vh[(size_t)t * d + i]);
                    hi = fmax(hi, vh[(size_t)t * d + i]);
                }
                const double tol = 1e-9 * fmax(fabs(lo), fabs(hi)) + 1e-300;
                CHECK(o >= lo - tol && o <= hi + tol);
            }
    }
    free(q);
    free(out);
    free(logits);
    free(mask);
    free(kh);
    free(vh);
}

static int run_cache(int kfmt, int vfmt, int rotate, int ch0, int n_sink, int W, int rope_w, int d)
{
    cache c;
    memset(&c, 0, sizeof(c));
    c.U = 3;
    c.d = d;
    c.cap = 512;
    c.n_sink = n_sink;
    c.kfmt = kfmt;
    c.rotate = rotate;
    c.ch0 = ch0;
    c.vfmt = vfmt;
    c.vclip = 0.92f;
    c.W = W;
    c.rope_w = rope_w;
    cache_alloc(&c);
    decode_and_check(&c, 0, 2, 0);
    int len = 0;
    while (len < c.cap) {
        int n = (rnd() % 4 == 0) ? (int)(rnd() % 200) + 1 : (int)(rnd() % 9) + 1;
        if (n > c.cap - len)
            n = c.cap - len;
        float *k = xalloc(sizeof(float) * c.U * n * d), *v = xalloc(sizeof(float) * c.U * n * d);
        for (int r = 0; r < c.U * n; r++)
            fill_token(&c, k + (size_t)r * d, v + (size_t)r * d);
        oracle_quant_append(CACHE_ARGS(&c), c.thr, c.U, len, n, k, v);
        free(k);
        free(v);
        len += n;
        if (rnd() % 4 == 0)
            decode_and_check(&c, len, 1 << (rnd() % 4), 0);
    }
    decode_and_check(&c, len, 8, 0);
    decode_and_check(&c, len, 4, 3); /* pruned: runs clean, outputs finite */
    cache_free(&c);
    return 1;
}

int main(void)
{
    check_conversions();
    check_transforms();
    int runs = 0;
    for (int kfmt = 0; kfmt < 4; kfmt++)
        for (int vfmt = 0; vfmt < 3; vfmt++) {
            const int rotate = kfmt == K_LLOYD4 ? (runs & 1) : 0;
            const int ch0 = kfmt != K_LLOYD4 ? (runs & 1) : 0;
            const int sinks[4] = {0, 1, 5, 64};
            const int windows[4] = {0, 64, 100, 256};
            const int d = (runs % 3 == 2) ? 64 : 128;
            runs += run_cache(kfmt, vfmt, rotate, ch0, sinks[runs % 4], windows[(runs / 2) % 4],
                              runs % 5 == 0 ? 128 : 0, d);
        }
    runs += run_cache(K_LLOYD4, V_KQV, 1, 0, 3, 1024, 256, 128); /* window above the capacity */
    runs += run_cache(K_ASYM2, V_INT2_TOKEN, 0, 1, 0, 1, 0, 64); /* window of one */
    printf("oracle_driver ok: %d caches\n", runs);
    return 0;
}
