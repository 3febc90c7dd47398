/*
 * kvq_oracle.c -- plain, slow, CPU reference for low-bit KV-cache decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the bench
 * use it.  It shares no code, header, table or constant generator with the HIP path.
 *
 * What it computes, and where the pages define it:
 *   - asymmetric INT-b keys/values with FP16 scale and zero per 32-channel group,
 *     channel 0 kept in BF16 and left out of the range estimate
 *       (Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV Caches, sec. 3.3
 *        and sec. C.3);
 *   - channel-major key storage so that decode can skip unselected rows (same, sec. 3.3);
 *   - Walsh-Hadamard rotation and a Lloyd-Max scalar codebook on keys
 *       (TurboQuant on Quantized Models, abstract and topic list; Statistical Inference
 *        and Quality Measures of KV Cache Quantisations Inspired by TurboQuant,
 *        "Quantisierungsschemata", scheme KQV, and "Theoretischer Rahmen" for the
 *        Beta -> Gaussian marginal that makes an N(0,1) codebook the right one);
 *   - BF16 sink tokens (TurboQuant on Quantized Models, abstract: sink-token preservation;
 *     Dual-QK sec. 3.3 / 4.1: first tokens kept in BF16);
 *   - a window of the most recent positions kept in BF16 and quantized only when they leave
 *     it (Dual-QK sec. 3.3 / 4.1: the most recent 256 entries stay BF16; TurboQuant on
 *     Quantized Models, abstract: past-only quantization, the current token attends
 *     unquantized);
 *   - dynamic query-channel-group pruning with one mask per GQA group, ranked by
 *     query energy summed over the group's heads (Dual-QK sec. 3.2, sec. C.2, App. A);
 *   - values as asymmetric INT4 per 32-channel group, or as per-token asymmetric INT2
 *     with a clipping ratio (Dual-QK sec. 3.3 and sec. B.2: per-token INT2 values with
 *     0.92 clipping), or KQV's value side: Walsh-Hadamard rotation, 3-bit Lloyd-Max codes
 *     with an FP16 norm and a 1-bit QJL sketch of the residual through a randomised
 *     Hadamard transform (KV-quantisation statistics, "Quantisierungsschemata" KQV and the
 *     QJL variance statement; TurboQuant on Quantized Models, abstract: SRHT-QJL);
 *   - attention over the decoded cache with one softmax over all positions
 *     (Dual-QK sec. 3.4: bucket scores share one global softmax);
 *   - bucket-relative RoPE (Dual-QK sec. 3.4 and C.4): keys, given with their rotary
 *     embedding at their absolute position, are stored relative to the anchor of their
 *     bucket of w positions, and the query is moved to each bucket's anchor the same way
 *     before it scores that bucket's keys (so each score is the one of the original
 *     keys); the pruning mask is taken per bucket.
 *
 * Precision.  The encoding (quantize + pack) runs in fp32 with a fixed operation order;
 * build with -ffp-contract=off and without fast-math so that every fp32 operation is a
 * single IEEE-754 round-to-nearest-even operation.  Decoding and attention run in fp64.
 *
 * Readings taken where the pages are silent are listed in the design notes; the ones
 * that change arithmetic are repeated at the function that implements them.
 *
 * Parity pins: every function here is checked by the CPU test-suite against something
 * other than itself (library conversions, explicit Hadamard matrices, brute-force code
 * search, exhaustive subset search, closed forms, published Lloyd-Max tables).
 */
#define _DEFAULT_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------ */
/* Format constants.  Key format ids: 0 = asymmetric INT2, 1 = asymmetric INT4,
 * 2 = 4-bit Lloyd-Max codebook, 3 = asymmetric INT8 (oracle only, for the convergence
 * check that 8-bit codes approach dense attention).  Value format ids: 0 = asymmetric INT4
 * per 32-channel group, 1 = per-token asymmetric INT2 with a clipping ratio.            */
enum { OK_ASYM2 = 0, OK_ASYM4 = 1, OK_LLOYD4 = 2, OK_ASYM8 = 3 };
enum { OV_ASYM4_G32 = 0, OV_ASYM2_TOKEN = 1, OV_KQV = 2 };

static int key_bits(int kfmt) { return kfmt == OK_ASYM2 ? 2 : kfmt == OK_ASYM8 ? 8 : 4; }

/* ------------------------------------------------------------------------------------ */
/* Conversions.  fp32 -> binary16 and fp32 -> bfloat16, both round-to-nearest-even,
 * written from the IEEE-754 definitions.                                                 */

uint16_t oracle_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ex = (x >> 23) & 0xFFu;
    uint32_t man = x & 0x7FFFFFu;
    if (ex == 0xFFu) /* inf or nan */
        return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    int e = (int)ex - 127 + 15; /* biased binary16 exponent */
    if (e >= 31)
        return (uint16_t)(sign | 0x7C00u);
    if (e >= 1) {
        /* normal result: keep 10 mantissa bits, round on the 13 dropped ones */
        uint32_t h = sign | ((uint32_t)e << 10) | (man >> 13);
        uint32_t rest = man & 0x1FFFu;
        if (rest > 0x1000u || (rest == 0x1000u && (h & 1u)))
            h += 1u; /* a carry into the exponent is the correct rounding, up to inf */
        return (uint16_t)h;
    }
    /* subnormal (or zero) result: value = m * 2^-24 with m = sig * 2^(ex-126) */
    if (ex == 0)
        return (uint16_t)sign; /* fp32 subnormals are far below half of 2^-24 */
    uint32_t sig = man | 0x800000u;
    int shift = 126 - (int)ex; /* >= 14 here */
    if (shift >= 25)
        return (uint16_t)sign; /* below or at half of the smallest subnormal: even = 0 */
    uint32_t m = sig >> shift;
    uint32_t rest = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rest > half || (rest == half && (m & 1u)))
        m += 1u; /* m may reach 1024, which is the smallest normal: still correct */
    return (uint16_t)(sign | m);
}

float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = ((uint32_t)h >> 10) & 0x1Fu;
    uint32_t m = (uint32_t)h & 0x3FFu;
    float out;
    if (e == 0) {
        /* zero or subnormal: m * 2^-24, exact in fp32 */
        out = (float)m * 5.9604644775390625e-08f;
        if (sign)
            out = -out;
        return out;
    }
    uint32_t x;
    if (e == 31)
        x = sign | 0x7F800000u | (m << 13);
    else
        x = sign | ((e - 15 + 127) << 23) | (m << 13);
    memcpy(&out, &x, 4);
    return out;
}

uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    if ((x & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((x >> 16) | 0x40u); /* quiet nan */
    uint32_t lsb = (x >> 16) & 1u;
    x += 0x7FFFu + lsb;
    return (uint16_t)(x >> 16);
}

float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t x = (uint32_t)b << 16;
    float f;
    memcpy(&f, &x, 4);
    return f;
}

/* array forms, for the conversion pins */
void oracle_f32_to_f16_array(const float *x, uint16_t *h, size_t n)
{
    for (size_t i = 0; i < n; i++)
        h[i] = oracle_f32_to_f16(x[i]);
}

void oracle_f16_to_f32_array(const uint16_t *h, float *x, size_t n)
{
    for (size_t i = 0; i < n; i++)
        x[i] = oracle_f16_to_f32(h[i]);
}

void oracle_f32_to_bf16_array(const float *x, uint16_t *h, size_t n)
{
    for (size_t i = 0; i < n; i++)
        h[i] = oracle_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------------------------------ */
/* Walsh-Hadamard transform, unnormalised Sylvester ordering, in place.  Stage h pairs
 * element j with j+h inside each block of 2h and writes (a+b, a-b), lower minus upper.
 * H*H = d*I, so the inverse is H/d.  (TurboQuant on Quantized Models: topic list,
 * Walsh-Hadamard transform; Statistical Inference ... TurboQuant: scheme KQV.)          */

void oracle_fwht_f32(float *y, int d)
{
    for (int h = 1; h < d; h <<= 1)
        for (int i = 0; i < d; i += 2 * h)
            for (int j = i; j < i + h; j++) {
                float a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
}

void oracle_fwht_f64(double *y, int d)
{
    for (int h = 1; h < d; h <<= 1)
        for (int i = 0; i < d; i += 2 * h)
            for (int j = i; j < i + h; j++) {
                double a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
}

/* Stride-halving tree sum in fp32: for h = n/2, n/4, ..., 1: a[i] += a[i+h] (i < h).
 * This fixed order is the one every fp32 sum of squares in the encoder and in the
 * pruning ranking uses.  n must be a power of two; a is clobbered.                      */
float oracle_tree_sum_f32(float *a, int n)
{
    for (int h = n / 2; h >= 1; h /= 2)
        for (int i = 0; i < h; i++)
            a[i] = a[i] + a[i + h];
    return a[0];
}

/* ------------------------------------------------------------------------------------ */
/* Lloyd-Max quantiser for N(0,1), symmetric, 2^bits levels, fp64.  Iterates the two
 * Lloyd conditions (thresholds at midpoints, centroids at conditional means) on the
 * positive half and mirrors it.  The conditional mean of N(0,1) on (a, b] is
 * (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  (Lloyd-Max codebook: TurboQuant on Quantized
 * Models, topic list; the N(0,1) target follows from the Beta((d-1)/2,(d-1)/2) ->
 * Gaussian marginal in Statistical Inference ... TurboQuant, "Theoretischer Rahmen".)
 * Writes cent[L] ascending and thr[L-1] = midpoints.  Returns iterations used.          */

static double npdf(double x) { return 0.39894228040143267794 * exp(-0.5 * x * x); }
/* upper tail Q(x) = 1 - Phi(x), accurate for x >= 0 */
static double nupper(double x) { return 0.5 * erfc(x * 0.70710678118654752440); }

int oracle_lloyd_max_gaussian(int levels, double tol, int max_iter, double *cent, double *thr)
{
    int half = levels / 2;
    double m[64], t[65];
    for (int i = 0; i < half; i++)
        m[i] = (i + 0.5) * (3.0 / half); /* spread over [0, 3] */
    int it;
    for (it = 0; it < max_iter; it++) {
        t[0] = 0.0;
        for (int i = 1; i < half; i++)
            t[i] = 0.5 * (m[i - 1] + m[i]);
        double delta = 0.0;
        for (int i = 0; i < half; i++) {
            double a = t[i];
            double mass, num;
            if (i + 1 < half) {
                double b = t[i + 1];
                mass = nupper(a) - nupper(b);
                num = npdf(a) - npdf(b);
            } else {
                mass = nupper(a);
                num = npdf(a);
            }
            double nm = num / mass;
            double dd = fabs(nm - m[i]);
            if (dd > delta)
                delta = dd;
            m[i] = nm;
        }
        if (delta < tol) {
            it++;
            break;
        }
    }
    for (int i = 0; i < half; i++) {
        cent[half + i] = m[i];
        cent[half - 1 - i] = -m[i];
    }
    for (int i = 0; i + 1 < levels; i++)
        thr[i] = 0.5 * (cent[i] + cent[i + 1]);
    return it;
}

/* ------------------------------------------------------------------------------------ */
/* Cache geometry shared by all entry points below.  Buffers are whole-cache host arrays
 * of U = batch * n_kv_heads units, indexed by absolute token position:
 *   k_codes u32 [U][R][cap]       R = d/16 (2-bit) | d/8 (4-bit) | d/4 (8-bit): row r of
 *                                 token t holds channels r*(32/b) .. ; channel
 *                                 r*(32/b)+j sits in bits [b*j, b*j+b-1]
 *   k_sz    u32 [U][d/32][cap]    asymmetric keys: low 16 bits fp16 scale, high fp16 zero
 *   k_norm  u16 [U][cap]          Lloyd-Max keys: fp16 rho
 *   k_ch0   u16 [U][cap]          protected channel 0: bf16
 *   v_codes u32 [U][cap/2][d/4]   INT4 values: word j of token pair P: bits [4k,4k+3] =
 *                                 channel 4j+k of token 2P, bits [16+4k, 16+4k+3] = same
 *                                 channel of 2P+1
 *           u32 [U][cap/2][d/8]   per-token INT2 values: word j of pair P: bits [2k,2k+1] =
 *                                 channel 8j+k of token 2P, bits [16+2k, 16+2k+1] = same
 *                                 channel of 2P+1
 *   v_sz    u32 [U][d/32][cap]    fp16 scale (low) / zero (high); one row ([U][1][cap])
 *                                 for per-token values
 *   sink_k  u16 [U][n_sink][d]    bf16 key in stored coordinates (rotated if rotation on)
 *   sink_v  u16 [U][n_sink][d]    bf16 value
 *   recent_k u16 [U][W][d]        recent window (W = n_recent > 0): ring slot t mod W holds
 *   recent_v u16 [U][W][d]        the bf16 key (stored coordinates) / value of position t
 *                                 while t is among the W most recent positions >= n_sink
 * Slots t < n_sink of the quantised arrays are never written, nor are those of positions
 * still in the recent window.                                                            */
typedef struct {
    int d, cap, n_sink, kfmt, rotate, ch0, vfmt;
    float vclip; /* per-token INT2 values: clipping ratio */
    int n_recent; /* W: most recent positions kept in BF16 (0: none) */
    uint32_t *k_codes, *k_sz, *v_codes, *v_sz;
    uint16_t *k_norm, *k_ch0, *sink_k, *sink_v, *recent_k, *recent_v;
    const float *cent, *thr; /* Lloyd-Max: 16 centroids, 15 thresholds (fp32) */
    int len; /* positions stored (decode: where the recent window starts) */
    int rope_w; /* bucket-relative RoPE: bucket width w (0: off) */
    const float *rope_cs; /* (cos, sin) of each bucket anchor's angles [bucket][d/2][2] */
    const float *vcent, *vthr; /* KQV values: 8 centroids, 7 thresholds (fp32) */
    const uint32_t *qjl; /* KQV values: the sketch's random signs, bit i set = channel i negated */
} ocache;

/* Bucket-relative RoPE (Dual-QK sec. 3.4 and C.4).  Reading: the rotary embedding pairs
 * channel i with channel i + d/2 (rotate-half layout), and a vector moved to the anchor of
 * bucket b is rotated back by that anchor's angles: with (cos, sin) = rope_cs[b][i],
 *   y_i <- y_i cos + y_{i+d/2} sin,   y_{i+d/2} <- y_{i+d/2} cos - y_i sin.
 * fp32 version: each product rounded, then the sum (this decides codes and masks).        */
static void anchor_back_f32(const ocache *c, int bucket, float *y)
{
    const int h = c->d / 2;
    const float *cs = c->rope_cs + (size_t)bucket * (size_t)c->d;
    for (int i = 0; i < h; i++) {
        float co = cs[2 * i], si = cs[2 * i + 1];
        float a = y[i], b = y[i + h];
        float p1 = a * co, p2 = b * si, p3 = b * co, p4 = a * si;
        y[i] = p1 + p2;
        y[i + h] = p3 - p4;
    }
}

/* The same rotation in fp64 (the query for the logits), from the same table entries. */
static void anchor_back_f64(const ocache *c, int bucket, double *y)
{
    const int h = c->d / 2;
    const float *cs = c->rope_cs + (size_t)bucket * (size_t)c->d;
    for (int i = 0; i < h; i++) {
        double co = (double)cs[2 * i], si = (double)cs[2 * i + 1];
        double a = y[i], b = y[i + h];
        y[i] = a * co + b * si;
        y[i + h] = b * co - a * si;
    }
}

static size_t krows(const ocache *c) { return (size_t)(c->d * key_bits(c->kfmt) / 32); }

/* Asymmetric INT-b quantisation of one group (Dual-QK sec. 3.3, "asymmetric INT2").
 * Reading: scale = (max-min)/(2^b-1) and zero = min, both stored as fp16, and the codes
 * are computed against the fp16-rounded values that decode will use; a group whose
 * range is zero (or whose fp16 scale is zero) codes to all zeros.  skip0 drops element 0
 * from the range estimate and codes it as 0 (channel-0 protection, Dual-QK sec. C.3).   */
static void asym_group(const float *x, int n, int bits, int skip0, uint8_t *code,
                       uint16_t *sh_out, uint16_t *zh_out)
{
    int qmax = (1 << bits) - 1;
    int first = skip0 ? 1 : 0;
    float mn = x[first], mx = x[first];
    for (int i = first + 1; i < n; i++) {
        if (x[i] < mn)
            mn = x[i];
        if (x[i] > mx)
            mx = x[i];
    }
    /* Reading: a zero minimum or range is taken as +0 (adding +0 turns -0 into +0 and
     * leaves every other value unchanged), so the stored fp16 sign bit never depends on
     * which of -0 / +0 a min/max scan meets first.                                      */
    mn = mn + 0.0f;
    float range = (mx - mn) + 0.0f;
    float scale32 = range / (float)qmax;
    uint16_t sh = oracle_f32_to_f16(scale32);
    uint16_t zh = oracle_f32_to_f16(mn);
    float sf = oracle_f16_to_f32(sh);
    float zf = oracle_f16_to_f32(zh);
    float inv = sf > 0.0f ? 1.0f / sf : 0.0f;
    for (int i = 0; i < n; i++) {
        if (i == 0 && skip0) {
            code[i] = 0;
            continue;
        }
        float diff = x[i] - zf;
        float u = diff * inv;
        float r = rintf(u);
        if (r < 0.0f)
            r = 0.0f;
        if (r > (float)qmax)
            r = (float)qmax;
        code[i] = (uint8_t)r;
    }
    *sh_out = sh;
    *zh_out = zh;
}

/* Per-token asymmetric INT2 of one value vector with clipping ratio `clip` (Dual-QK
 * sec. B.2: values use per-token asymmetric INT2 with a 0.92 clipping ratio).
 * Reading: the clipped range is [clip*min, clip*max] (both ends scaled toward zero, the
 * usual convention of rotation-based quantizers for a clipping ratio); scale = clipped
 * range / 3 and zero = clip*min as fp16, codes against the rounded values as in
 * asym_group, so entries outside the clipped range saturate at code 0 or 3.  With clip = 1
 * this is asym_group over the whole vector.                                              */
static void asym_token_clip(const float *x, int n, float clip, uint8_t *code, uint16_t *sh_out,
                            uint16_t *zh_out)
{
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; i++) {
        if (x[i] < mn)
            mn = x[i];
        if (x[i] > mx)
            mx = x[i];
    }
    mn = clip * mn + 0.0f;
    mx = clip * mx;
    float range = (mx - mn) + 0.0f;
    float scale32 = range / 3.0f;
    uint16_t sh = oracle_f32_to_f16(scale32);
    uint16_t zh = oracle_f32_to_f16(mn);
    float sf = oracle_f16_to_f32(sh);
    float zf = oracle_f16_to_f32(zh);
    float inv = sf > 0.0f ? 1.0f / sf : 0.0f;
    for (int i = 0; i < n; i++) {
        float diff = x[i] - zf;
        float u = diff * inv;
        float r = rintf(u);
        if (r < 0.0f)
            r = 0.0f;
        if (r > 3.0f)
            r = 3.0f;
        code[i] = (uint8_t)r;
    }
    *sh_out = sh;
    *zh_out = zh;
}

/* Quantise and store the key y (stored coordinates: already rotated when rotation is on)
 * and the value v of position t of unit u; d fp32 values each.                          */
static void quant_stored(const ocache *c, size_t u, int t, const float *y, const float *v)
{
    const int d = c->d;
    const size_t cap = (size_t)c->cap;
    uint8_t code[256];
    const int kb = key_bits(c->kfmt);
    if (c->kfmt == OK_LLOYD4) {
        /* rho = RMS of the stored coordinates (= ||k|| when rotated), fp16; z = y / rho;
         * code = number of thresholds strictly below z.                                  */
        float sq[256];
        for (int i = 0; i < d; i++)
            sq[i] = y[i] * y[i];
        float s2 = oracle_tree_sum_f32(sq, d);
        float rho32 = sqrtf(s2 / (float)d);
        uint16_t rh = oracle_f32_to_f16(rho32);
        float rf = oracle_f16_to_f32(rh);
        float inv = rf > 0.0f ? 1.0f / rf : 0.0f;
        for (int i = 0; i < d; i++) {
            float z = y[i] * inv;
            int cnt = 0;
            for (int j = 0; j < 15; j++)
                if (z > c->thr[j])
                    cnt++;
            code[i] = (uint8_t)cnt;
        }
        c->k_norm[u * cap + (size_t)t] = rh;
    } else {
        for (int g = 0; g < d / 32; g++) {
            uint16_t sh, zh;
            asym_group(y + 32 * g, 32, kb, (g == 0 && c->ch0), code + 32 * g, &sh, &zh);
            c->k_sz[(u * (size_t)(d / 32) + (size_t)g) * cap + (size_t)t] =
                (uint32_t)sh | ((uint32_t)zh << 16);
        }
        if (c->ch0)
            c->k_ch0[u * cap + (size_t)t] = oracle_f32_to_bf16(y[0]);
    }
    /* channel-major rows: row r holds 32/kb channels of this token */
    const int per = 32 / kb;
    const size_t R = krows(c);
    for (size_t r = 0; r < R; r++) {
        uint32_t w = 0;
        for (int j = 0; j < per; j++)
            w |= (uint32_t)code[(int)r * per + j] << (kb * j);
        c->k_codes[(u * R + r) * cap + (size_t)t] = w;
    }

    uint8_t vc[256];
    if (c->vfmt == OV_KQV) {
        /* KQV values (KV-quantisation statistics, "Quantisierungsschemata": WHT, (n-1)-bit
         * scalar MSE codes, 1-bit QJL sketch of the residual; TurboQuant on Quantized Models:
         * the sketch matrix is a randomised Hadamard transform S = H D).  fp32 throughout:
         *   y = FWHT(v); rho = fp16(sqrt(tree_sum(y^2) / d)); z = y / rho; code = number of
         *   the 7 thresholds strictly below z; y^ = rho * cent[code]; r = y - y^;
         *   sketch bit i = 1 when (H D r)_i < 0; gamma = fp16(sqrt(tree_sum(r^2))).
         * Stored: nibble i = code_i | bit_i << 3 in the INT4 pair layout; v_sz = rho | gamma<<16. */
        float y2[256], sq[256], r[256], w[256];
        memcpy(y2, v, sizeof(float) * (size_t)d);
        oracle_fwht_f32(y2, d);
        for (int i = 0; i < d; i++)
            sq[i] = y2[i] * y2[i];
        float s2 = oracle_tree_sum_f32(sq, d);
        uint16_t rh = oracle_f32_to_f16(sqrtf(s2 / (float)d));
        float rf = oracle_f16_to_f32(rh);
        float inv = rf > 0.0f ? 1.0f / rf : 0.0f;
        for (int i = 0; i < d; i++) {
            float z = y2[i] * inv;
            int cnt = 0;
            for (int j = 0; j < 7; j++)
                if (z > c->vthr[j])
                    cnt++;
            vc[i] = (uint8_t)cnt;
            float yh = rf * c->vcent[cnt];
            r[i] = y2[i] - yh;
            w[i] = ((c->qjl[i / 32] >> (i % 32)) & 1u) ? -r[i] : r[i];
            sq[i] = r[i] * r[i];
        }
        oracle_fwht_f32(w, d);
        float g2 = oracle_tree_sum_f32(sq, d);
        uint16_t gh = oracle_f32_to_f16(sqrtf(g2));
        for (int i = 0; i < d; i++)
            vc[i] |= (uint8_t)((w[i] < 0.0f ? 1u : 0u) << 3);
        c->v_sz[u * cap + (size_t)t] = (uint32_t)rh | ((uint32_t)gh << 16);
        const size_t W4 = (size_t)(d / 4);
        uint32_t *prow = c->v_codes + (u * (cap / 2) + (size_t)(t / 2)) * W4;
        const int s16 = (t & 1) ? 16 : 0;
        for (size_t j = 0; j < W4; j++) {
            uint32_t half = 0;
            for (int k2 = 0; k2 < 4; k2++)
                half |= (uint32_t)vc[4 * j + (size_t)k2] << (4 * k2);
            prow[j] = (prow[j] & ~(0xFFFFu << s16)) | (half << s16);
        }
        return;
    }
    if (c->vfmt == OV_ASYM2_TOKEN) {
        /* values: per-token asymmetric INT2 with clipping, pair-interleaved words */
        uint16_t sh, zh;
        asym_token_clip(v, d, c->vclip, vc, &sh, &zh);
        c->v_sz[u * cap + (size_t)t] = (uint32_t)sh | ((uint32_t)zh << 16);
        const size_t W2 = (size_t)(d / 8);
        uint32_t *row2 = c->v_codes + (u * (cap / 2) + (size_t)(t / 2)) * W2;
        const int s16 = (t & 1) ? 16 : 0;
        for (size_t j = 0; j < W2; j++) {
            uint32_t half = 0;
            for (int k2 = 0; k2 < 8; k2++)
                half |= (uint32_t)vc[8 * j + (size_t)k2] << (2 * k2);
            row2[j] = (row2[j] & ~(0xFFFFu << s16)) | (half << s16);
        }
        return;
    }
    /* values: asymmetric INT4 per 32-channel group, no channel exclusion */
    for (int g = 0; g < d / 32; g++) {
        uint16_t sh, zh;
        asym_group(v + 32 * g, 32, 4, 0, vc + 32 * g, &sh, &zh);
        c->v_sz[(u * (size_t)(d / 32) + (size_t)g) * cap + (size_t)t] =
            (uint32_t)sh | ((uint32_t)zh << 16);
    }
    const size_t W = (size_t)(d / 4);
    uint32_t *pairrow = c->v_codes + (u * (cap / 2) + (size_t)(t / 2)) * W;
    const int sh16 = (t & 1) ? 16 : 0;
    for (size_t j = 0; j < W; j++) {
        uint32_t half = 0;
        for (int k2 = 0; k2 < 4; k2++)
            half |= (uint32_t)vc[4 * j + (size_t)k2] << (4 * k2);
        pairrow[j] = (pairrow[j] & ~(0xFFFFu << sh16)) | (half << sh16);
    }
}

/* Store one token (K and V) at absolute position t of unit u; k and v are d fp32 values.
 * The key goes to stored coordinates first (FWHT when rotation is on).  Positions below
 * n_sink are kept in BF16.  Without a recent window every other position is quantised at
 * once.  With a window of W positions (reading of Dual-QK sec. 3.3 / 4.1 and of past-only
 * quantization), a position enters ring slot t mod W as BF16 and is quantised only when the
 * position t + W takes its slot, from that BF16 copy -- so with a window the codes of a
 * position never depend on how the appends were cut.                                    */
static void quant_token(const ocache *c, size_t u, int t, const float *k, const float *v)
{
    const int d = c->d;
    float y[256];
    memcpy(y, k, sizeof(float) * (size_t)d);
    if (c->rope_w > 0)
        anchor_back_f32(c, t / c->rope_w, y);
    if (c->rotate)
        oracle_fwht_f32(y, d);

    if (t < c->n_sink) {
        /* Sink token: BF16 key (in stored coordinates) and BF16 value.
         * (TurboQuant on Quantized Models: sink-token preservation.)                    */
        uint16_t *sk = c->sink_k + (u * (size_t)c->n_sink + (size_t)t) * (size_t)d;
        uint16_t *sv = c->sink_v + (u * (size_t)c->n_sink + (size_t)t) * (size_t)d;
        for (int i = 0; i < d; i++) {
            sk[i] = oracle_f32_to_bf16(y[i]);
            sv[i] = oracle_f32_to_bf16(v[i]);
        }
        return;
    }
    if (c->n_recent == 0) {
        quant_stored(c, u, t, y, v);
        return;
    }
    const size_t W = (size_t)c->n_recent;
    uint16_t *rk = c->recent_k + (u * W + (size_t)t % W) * (size_t)d;
    uint16_t *rv = c->recent_v + (u * W + (size_t)t % W) * (size_t)d;
    if (t - (int)W >= c->n_sink) {
        /* position t - W leaves the window: quantise its BF16 copy */
        float ok[256], ov[256];
        for (int i = 0; i < d; i++) {
            ok[i] = oracle_bf16_to_f32(rk[i]);
            ov[i] = oracle_bf16_to_f32(rv[i]);
        }
        quant_stored(c, u, t - (int)W, ok, ov);
    }
    for (int i = 0; i < d; i++) {
        rk[i] = oracle_f32_to_bf16(y[i]);
        rv[i] = oracle_f32_to_bf16(v[i]);
    }
}

/* Append n_new tokens per unit at positions [t0, t0+n_new) for units [0, n_units).
 * k_new, v_new: fp32 [n_units][n_new][d].  OpenMP over units.                            */
void oracle_quant_append(int d, int cap, int n_sink, int kfmt, int rotate, int ch0, int vfmt, float vclip,
                         int n_recent,
                         uint32_t *k_codes, uint32_t *k_sz, uint16_t *k_norm, uint16_t *k_ch0,
                         uint32_t *v_codes, uint32_t *v_sz, uint16_t *sink_k, uint16_t *sink_v,
                         uint16_t *recent_k, uint16_t *recent_v, int rope_w, const float *rope_cs,
                         const float *vcent, const float *vthr, const uint32_t *qjl,
                         const float *cent, const float *thr, int n_units, int t0, int n_new,
                         const float *k_new, const float *v_new)
{
    ocache c = {d, cap, n_sink, kfmt, rotate, ch0, vfmt, vclip, n_recent, k_codes, k_sz, v_codes, v_sz,
                k_norm, k_ch0, sink_k, sink_v, recent_k, recent_v, cent, thr, t0 + n_new, rope_w, rope_cs, vcent, vthr, qjl};
#pragma omp parallel for schedule(static)
    for (int u = 0; u < n_units; u++)
        for (int i = 0; i < n_new; i++) {
            size_t off = ((size_t)u * (size_t)n_new + (size_t)i) * (size_t)d;
            quant_token(&c, (size_t)u, t0 + i, k_new + off, v_new + off);
        }
}

/* ------------------------------------------------------------------------------------ */
/* Query-channel-group pruning mask (Dual-QK sec. 3.2 and sec. C.2): groups of 16
 * channels of the stored key coordinates; energy of group p for head h is the fp32
 * tree sum of qt^2 over its 16 channels; the group score sums the G heads of the GQA
 * group in ascending head order; keep the m highest scores, ties to the lower index.
 * qt: fp32 [G][d] query in stored coordinates.  m <= 0 or m >= d/16 keeps everything.
 * Returns a bit mask, bit p = group p kept.                                              */
uint32_t oracle_prune_mask(const float *qt, int G, int d, int m)
{
    const int P = d / 16;
    uint32_t all = (P >= 32) ? 0xFFFFFFFFu : ((1u << P) - 1u);
    if (m <= 0 || m >= P)
        return all;
    float E[16];
    for (int p = 0; p < P; p++) {
        float acc = 0.0f;
        for (int h = 0; h < G; h++) {
            float sq[16];
            for (int i = 0; i < 16; i++) {
                float qv = qt[(size_t)h * (size_t)d + (size_t)(16 * p + i)];
                sq[i] = qv * qv;
            }
            float e = oracle_tree_sum_f32(sq, 16);
            acc = (h == 0) ? e : acc + e;
        }
        E[p] = acc;
    }
    uint32_t mask = 0;
    for (int p = 0; p < P; p++) {
        int rank = 0;
        for (int o = 0; o < P; o++)
            if (E[o] > E[p] || (E[o] == E[p] && o < p))
                rank++;
        if (rank < m)
            mask |= 1u << p;
    }
    return mask;
}

/* ------------------------------------------------------------------------------------ */
/* Decoding of stored tokens into fp64 (stored coordinates).                             */

/* Position t (< len) is still in the recent window: held in BF16 in ring slot t mod W. */
static int in_window(const ocache *c, int t)
{
    return c->n_recent > 0 && t >= c->n_sink && t >= c->len - c->n_recent;
}

static void decode_key(const ocache *c, size_t u, int t, double *kh)
{
    const int d = c->d;
    const size_t cap = (size_t)c->cap;
    if (t < c->n_sink) {
        const uint16_t *sk = c->sink_k + (u * (size_t)c->n_sink + (size_t)t) * (size_t)d;
        for (int i = 0; i < d; i++)
            kh[i] = (double)oracle_bf16_to_f32(sk[i]);
        return;
    }
    if (in_window(c, t)) {
        const size_t W = (size_t)c->n_recent;
        const uint16_t *rk = c->recent_k + (u * W + (size_t)t % W) * (size_t)d;
        for (int i = 0; i < d; i++)
            kh[i] = (double)oracle_bf16_to_f32(rk[i]);
        return;
    }
    const int kb = key_bits(c->kfmt);
    const int per = 32 / kb;
    const size_t R = krows(c);
    const uint32_t msk = (kb == 32) ? 0xFFFFFFFFu : ((1u << kb) - 1u);
    int code[256];
    for (size_t r = 0; r < R; r++) {
        uint32_t w = c->k_codes[(u * R + r) * cap + (size_t)t];
        for (int j = 0; j < per; j++)
            code[(int)r * per + j] = (int)((w >> (kb * j)) & msk);
    }
    if (c->kfmt == OK_LLOYD4) {
        double rf = (double)oracle_f16_to_f32(c->k_norm[u * cap + (size_t)t]);
        for (int i = 0; i < d; i++)
            kh[i] = rf * (double)c->cent[code[i]];
        return;
    }
    for (int g = 0; g < d / 32; g++) {
        uint32_t sz = c->k_sz[(u * (size_t)(d / 32) + (size_t)g) * cap + (size_t)t];
        double sf = (double)oracle_f16_to_f32((uint16_t)(sz & 0xFFFFu));
        double zf = (double)oracle_f16_to_f32((uint16_t)(sz >> 16));
        for (int i = 0; i < 32; i++)
            kh[32 * g + i] = (double)code[32 * g + i] * sf + zf;
    }
    if (c->ch0)
        kh[0] = (double)oracle_bf16_to_f32(c->k_ch0[u * cap + (size_t)t]);
}

static void decode_value(const ocache *c, size_t u, int t, double *vh)
{
    const int d = c->d;
    const size_t cap = (size_t)c->cap;
    if (t < c->n_sink) {
        const uint16_t *sv = c->sink_v + (u * (size_t)c->n_sink + (size_t)t) * (size_t)d;
        for (int i = 0; i < d; i++)
            vh[i] = (double)oracle_bf16_to_f32(sv[i]);
        return;
    }
    if (in_window(c, t)) {
        const size_t W = (size_t)c->n_recent;
        const uint16_t *rv = c->recent_v + (u * W + (size_t)t % W) * (size_t)d;
        for (int i = 0; i < d; i++)
            vh[i] = (double)oracle_bf16_to_f32(rv[i]);
        return;
    }
    const int sh16 = (t & 1) ? 16 : 0;
    if (c->vfmt == OV_KQV) {
        /* y~ = rho cent[code] + sqrt(pi/2)/d * gamma * D H sigma (sigma_i = -1 for a set
         * sketch bit: S^T sign(S r) with S = H D), then v^ = H y~ / d.  fp64.              */
        const uint32_t *prow = c->v_codes + (u * (cap / 2) + (size_t)(t / 2)) * (size_t)(d / 4);
        uint32_t sz = c->v_sz[u * cap + (size_t)t];
        double rf = (double)oracle_f16_to_f32((uint16_t)(sz & 0xFFFFu));
        double gf = (double)oracle_f16_to_f32((uint16_t)(sz >> 16));
        double hs[256];
        for (int i = 0; i < d; i++) {
            int nib = (int)(((prow[i / 4] >> sh16) >> (4 * (i % 4))) & 0xFu);
            vh[i] = rf * (double)c->vcent[nib & 7];
            hs[i] = (nib & 8) ? -1.0 : 1.0;
        }
        oracle_fwht_f64(hs, d);
        const double k = sqrt(M_PI / 2.0) / (double)d * gf;
        for (int i = 0; i < d; i++)
            vh[i] += k * (((c->qjl[i / 32] >> (i % 32)) & 1u) ? -hs[i] : hs[i]);
        oracle_fwht_f64(vh, d);
        for (int i = 0; i < d; i++)
            vh[i] /= (double)d;
        return;
    }
    if (c->vfmt == OV_ASYM2_TOKEN) {
        const uint32_t *row2 = c->v_codes + (u * (cap / 2) + (size_t)(t / 2)) * (size_t)(d / 8);
        uint32_t sz = c->v_sz[u * cap + (size_t)t];
        double sf = (double)oracle_f16_to_f32((uint16_t)(sz & 0xFFFFu));
        double zf = (double)oracle_f16_to_f32((uint16_t)(sz >> 16));
        for (int i = 0; i < d; i++) {
            int cd = (int)(((row2[i / 8] >> sh16) >> (2 * (i % 8))) & 0x3u);
            vh[i] = (double)cd * sf + zf;
        }
        return;
    }
    const size_t W = (size_t)(d / 4);
    const uint32_t *pairrow = c->v_codes + (u * (cap / 2) + (size_t)(t / 2)) * W;
    for (int g = 0; g < d / 32; g++) {
        uint32_t sz = c->v_sz[(u * (size_t)(d / 32) + (size_t)g) * cap + (size_t)t];
        double sf = (double)oracle_f16_to_f32((uint16_t)(sz & 0xFFFFu));
        double zf = (double)oracle_f16_to_f32((uint16_t)(sz >> 16));
        for (int i = 32 * g; i < 32 * g + 32; i++) {
            uint32_t w = pairrow[i / 4] >> sh16;
            int cd = (int)((w >> (4 * (i % 4))) & 0xFu);
            vh[i] = (double)cd * sf + zf;
        }
    }
}

/* Decoded cache of one unit, for tests: keys in stored coordinates, values. [len][d]. */
void oracle_dequant_unit(int d, int cap, int n_sink, int kfmt, int rotate, int ch0, int vfmt, float vclip,
                         int n_recent,
                         uint32_t *k_codes, uint32_t *k_sz, uint16_t *k_norm, uint16_t *k_ch0,
                         uint32_t *v_codes, uint32_t *v_sz, uint16_t *sink_k, uint16_t *sink_v,
                         uint16_t *recent_k, uint16_t *recent_v, int rope_w, const float *rope_cs,
                         const float *vcent, const float *vthr, const uint32_t *qjl,
                         const float *cent, int unit, int len, double *kh, double *vh)
{
    ocache c = {d, cap, n_sink, kfmt, rotate, ch0, vfmt, vclip, n_recent, k_codes, k_sz, v_codes, v_sz,
                k_norm, k_ch0, sink_k, sink_v, recent_k, recent_v, cent, 0, len, rope_w, rope_cs, vcent, vthr, qjl};
    for (int t = 0; t < len; t++) {
        decode_key(&c, (size_t)unit, t, kh + (size_t)t * (size_t)d);
        decode_value(&c, (size_t)unit, t, vh + (size_t)t * (size_t)d);
    }
}

/* ------------------------------------------------------------------------------------ */
/* Decode attention for units [0, n_units) (OpenMP over units).
 * q: fp32 [n_units][G][d] raw query (G = query heads of the unit's GQA group; query head
 *    h of a sequence reads KV head floor(h/G), so the G rows of a unit are consecutive).
 * For each head: logits l_t = sm * sum_{c kept} qs_c * k^_{t,c} / d_rot over t in [0, len),
 * where qs is the query in stored coordinates (FWHT(q) when keys are rotated, then
 * d_rot = d; otherwise qs = q and d_rot = 1), k^ the decoded stored key; p = softmax(l);
 * out = sum_t p_t v^_t.  All in fp64, two passes (max, then exp and sums).
 * The mask is computed from the fp32 stored-coordinate query (oracle_prune_mask) and
 * written to mask_out[u] when mask_out is not null.  With bucket-relative RoPE (rope_w > 0)
 * the query is moved to each bucket's anchor first, in fp32 for the mask and in fp64 for the
 * logits, so every bucket b < ceil(len / w) has its own query and mask, written to
 * mask_out[u * ceil(cap / w) + b]; position t is scored in bucket t / w.  logits_out (nullable) receives the
 * fp64 logits [n_units][G][len].                                                         */
void oracle_decode_attn(int d, int cap, int n_sink, int kfmt, int rotate, int ch0, int vfmt, float vclip,
                         int n_recent,
                        uint32_t *k_codes, uint32_t *k_sz, uint16_t *k_norm, uint16_t *k_ch0,
                        uint32_t *v_codes, uint32_t *v_sz, uint16_t *sink_k, uint16_t *sink_v,
                         uint16_t *recent_k, uint16_t *recent_v, int rope_w, const float *rope_cs,
                         const float *vcent, const float *vthr, const uint32_t *qjl,
                        const float *cent, int n_units, int len, int G, const float *q,
                        double sm, int keep_groups, double *out, uint8_t *mask_out,
                        double *logits_out)
{
    ocache c = {d, cap, n_sink, kfmt, rotate, ch0, vfmt, vclip, n_recent, k_codes, k_sz, v_codes, v_sz,
                k_norm, k_ch0, sink_k, sink_v, recent_k, recent_v, cent, 0, len, rope_w, rope_cs, vcent, vthr, qjl};
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < n_units; u++) {
        const float *qu = q + (size_t)u * (size_t)G * (size_t)d;
        /* one query per bucket (one bucket without RoPE): the fp32 stored-coordinate query
         * for the bucket's mask, and the fp64 one for its logits                          */
        const int nbq = (rope_w > 0 && len > 0) ? (len + rope_w - 1) / rope_w : 1;
        float *qt32 = (float *)malloc(sizeof(float) * (size_t)G * (size_t)d);
        double *qs = (double *)malloc(sizeof(double) * (size_t)nbq * (size_t)G * (size_t)d);
        uint32_t *masks = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)nbq);
        double *lg = (double *)malloc(sizeof(double) * (size_t)G * (size_t)(len > 0 ? len : 1));
        double kh[256], vh[256];
        for (int bq = 0; bq < nbq; bq++) {
            for (int h = 0; h < G; h++) {
                float *q32 = qt32 + (size_t)h * (size_t)d;
                double *q64 = qs + ((size_t)bq * (size_t)G + (size_t)h) * (size_t)d;
                memcpy(q32, qu + (size_t)h * (size_t)d, sizeof(float) * (size_t)d);
                for (int i = 0; i < d; i++)
                    q64[i] = (double)q32[i];
                if (rope_w > 0) {
                    anchor_back_f32(&c, bq, q32);
                    anchor_back_f64(&c, bq, q64);
                }
                if (rotate) {
                    oracle_fwht_f32(q32, d);
                    oracle_fwht_f64(q64, d);
                }
            }
            masks[bq] = oracle_prune_mask(qt32, G, d, keep_groups);
            if (mask_out) {
                const int n_rb = rope_w > 0 ? (cap + rope_w - 1) / rope_w : 1;
                mask_out[(size_t)u * (size_t)n_rb + (size_t)bq] = (uint8_t)masks[bq];
            }
        }
        const double scale = sm / (rotate ? (double)d : 1.0);
        /* pass 1: logits, each position against its bucket's query and mask */
        for (int t = 0; t < len; t++) {
            decode_key(&c, (size_t)u, t, kh);
            const int bq = rope_w > 0 ? t / rope_w : 0;
            const uint32_t mask = masks[bq];
            for (int h = 0; h < G; h++) {
                const double *q64 = qs + ((size_t)bq * (size_t)G + (size_t)h) * (size_t)d;
                double s = 0.0;
                for (int i = 0; i < d; i++)
                    if (mask & (1u << (i / 16)))
                        s += q64[i] * kh[i];
                lg[(size_t)h * (size_t)len + (size_t)t] = scale * s;
            }
        }
        if (logits_out)
            memcpy(logits_out + (size_t)u * (size_t)G * (size_t)len, lg,
                   sizeof(double) * (size_t)G * (size_t)len);
        /* pass 2: softmax-weighted values */
        double mx[64], den[64];
        for (int h = 0; h < G; h++) {
            mx[h] = -INFINITY;
            for (int t = 0; t < len; t++)
                if (lg[(size_t)h * (size_t)len + (size_t)t] > mx[h])
                    mx[h] = lg[(size_t)h * (size_t)len + (size_t)t];
            den[h] = 0.0;
        }
        double *o = out + (size_t)u * (size_t)G * (size_t)d;
        for (size_t i = 0; i < (size_t)G * (size_t)d; i++)
            o[i] = 0.0;
        for (int t = 0; t < len; t++) {
            decode_value(&c, (size_t)u, t, vh);
            for (int h = 0; h < G; h++) {
                double p = exp(lg[(size_t)h * (size_t)len + (size_t)t] - mx[h]);
                den[h] += p;
                for (int i = 0; i < d; i++)
                    o[(size_t)h * (size_t)d + (size_t)i] += p * vh[i];
            }
        }
        for (int h = 0; h < G; h++)
            for (int i = 0; i < d; i++)
                o[(size_t)h * (size_t)d + (size_t)i] = len > 0 ? o[(size_t)h * (size_t)d + (size_t)i] / den[h] : 0.0;
        free(qt32);
        free(qs);
        free(masks);
        free(lg);
    }
}

/* Thread count of the OpenMP loops (the benchmark times the oracle with all host threads
 * and with one); no arithmetic depends on it. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
