// kvq_decode.hip -- decode attention scored straight from the packed low-bit cache.
//
// What it computes (the pages this library implements):
//   * logits from packed key codes without decompressing keys (TurboQuant on Quantized
//     Models, abstract: fused scoring against codes); for asymmetric keys
//       l_t = sm * sum_g [ s_g * sum_{c in g} q_c code_c + z_g * sum_{c in g} q_c ]
//             (+ q_0 k_0 for the BF16 channel 0, Dual-QK sec. 3.3 / C.3),
//     for Lloyd-Max keys l_t = sm / d_rot * rho_t * sum_c q~_c cent[code_c] with q~ the
//     query in the keys' rotated coordinates (Walsh-Hadamard, TurboQuant topic list);
//   * an optional per-GQA-group channel mask from the current queries (Dual-QK sec. 3.2,
//     C.2): only the kept 16-channel key rows are loaded (channel-major rows, sec. 3.3);
//   * one softmax over all positions (Dual-QK sec. 3.4), computed online per split and
//     merged across splits by the last workgroup of each (sequence, KV head);
//   * values from INT4 codes: o = sum_t p_t s_{t,g} code_{t,c} + sum_t p_t z_{t,g}.
//
// MI355X mapping (one workgroup = 4 waves = one context split of one unit):
//   * score phase, lane per position: each lane scores 4 consecutive positions; a key row
//     is one dwordx4 load per lane (64 lanes read 1 KiB contiguous).  Asymmetric codes are
//     spread into bytes by shift+mask and multiplied with v_dot4_i32_i8 against the query
//     held as a 16-bit integer in two signed-byte planes (SGPRs): exact int32 sums, and the
//     zero-point term uses the same integer query, so code and zero terms together equal
//     q_int . k^ with no cancellation between them (heavy-tailed keys make the group zero
//     large).  Lloyd-Max codes go through an LDS table of fp16 centroid pairs and
//     v_dot2_f32_f16 against fp16 query pairs.
//   * value phase, lane per channel: each lane owns 16 channels and accumulates with
//     v_dot2_f32_f16 over position pairs (value words interleave two positions), taking
//     the fp16 weights p*s of each position pair from LDS.
//   * no MFMA: this is a bandwidth-bound scan.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int D, int G, int KF>
struct Cfg {
    static constexpr int KB = (KF == KVQ_K_ASYM2) ? 2 : 4;
    static constexpr int KROWS = D * KB / 32;      // key code rows (words per position)
    static constexpr int PPW = 16 / KB;            // fp16 pairs per key word (Lloyd-Max)
    static constexpr int NREG = 8 / KB;            // byte-spread registers per key word (asym)
    static constexpr int NG = D / 32;              // scale groups
    static constexpr int NP = D / 16;              // prune groups
    static constexpr int RPP = 16 * KB / 32;       // key rows per prune group
    static constexpr int TPL = 4;                  // positions per lane in the score phase
    static constexpr int TILE = 64 * TPL;
    static constexpr int WPP = D / 4;              // value words per position pair
    static constexpr int LPP = WPP / 4;            // value lanes per pair (dwordx4 each)
    static constexpr int PPI = 64 / LPP;           // pairs per value iteration
    static constexpr int PAIRS = TILE / 2;
    static constexpr int VIT = PAIRS / PPI;
    static constexpr int WSTRIDE = NG * G;         // u32 weights per pair in LDS
    static constexpr int CPL = D / 64;             // channels per lane in the prologue
    static_assert(TILE == kTile, "host and device tile must agree");
};

// Unnormalised Walsh-Hadamard transform across the wave (stage order h = 1, 2, 4, ...).
template <int CPL>
__device__ __forceinline__ void fwht_wave(float (&y)[CPL], int lane)
{
    if constexpr (CPL == 2) {
        float a = y[0], b = y[1];
        y[0] = a + b;
        y[1] = a - b;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            float other = __shfl_xor(y[s], m);
            y[s] = (lane & m) ? other - y[s] : y[s] + other;
        }
    }
}

template <int D, int G, int KF>
struct Smem {
    using C = Cfg<D, G, KF>;
    float q[G][D];                                  // stored-coordinate query (scaled)
    float e[G][C::NP];                              // group energies
    float amax[G][C::NP];                           // group max |q~|
    uint32_t qp[C::KROWS][G][8];                    // per key row: fp16 query pairs (Lloyd-Max)
                                                    // or int8 hi/lo query planes (asym)
    float qz[G][C::NG];                             // zero-term integer query sums
    float q0[G];                                    // channel-0 coefficient (integer units)
    float qsc[G];                                   // integer query unit, log2 logit units
    uint32_t lut[KF == KVQ_K_LLOYD4 ? 256 : 1];     // Lloyd-Max code-pair table (fp16x2)
    float sink_p[G][kMaxSink];
    union {
        uint32_t w[kWavesPerBlock][C::PAIRS][C::WSTRIDE]; // fp16 weight pairs per wave
        float merge[kWavesPerBlock][G][D + 2];            // per-wave (m, l, o)
    } u;
    int last;
};

template <int D, int G, int KF>
__global__ __launch_bounds__(kBlock) void decode_kernel(DecodeParams p)
{
    using C = Cfg<D, G, KF>;
    constexpr int KB = C::KB, KROWS = C::KROWS, PPW = C::PPW, NG = C::NG, NP = C::NP;
    constexpr int TPL = C::TPL, TILE = C::TILE, WPP = C::WPP, LPP = C::LPP, PPI = C::PPI;
    constexpr int VIT = C::VIT, CPL = C::CPL;
    __shared__ Smem<D, G, KF> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int split = blockIdx.x;
    const int unit = blockIdx.y;
    const int b = unit / p.n_kv_heads;
    const int kvh = unit % p.n_kv_heads;
    const size_t cap = (size_t)p.cap;
    const int n_q_heads = p.n_kv_heads * G;

    // ------------------------------------------------------------------ prologue
    // phase 1: each wave prepares heads h = wave, wave + 4, ...: fp32 query in stored
    // coordinates (FWHT when keys are rotated), 16-channel group energies and max |q|.
    for (int h = wave; h < G; h += kWavesPerBlock) {
        const size_t qoff = ((size_t)b * n_q_heads + (size_t)kvh * G + h) * D + (size_t)lane * CPL;
        float y[CPL];
        if (p.q_bf16) {
            const uint16_t *qb = static_cast<const uint16_t *>(p.q) + qoff;
#pragma unroll
            for (int s = 0; s < CPL; s++)
                y[s] = bf16_to_f32(qb[s]);
        } else {
            const float *qf = static_cast<const float *>(p.q) + qoff;
#pragma unroll
            for (int s = 0; s < CPL; s++)
                y[s] = qf[s];
        }
        if (p.rotate)
            fwht_wave<CPL>(y, lane);
        float sq[CPL], am = 0.0f;
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            sm.q[h][lane * CPL + s] = y[s];
            sq[s] = y[s] * y[s];
            am = fmaxf(am, fabsf(y[s]));
        }
        // stride-halving tree over the 16 channels of a group: lanes of one group are
        // 16/CPL consecutive lanes; the xor butterfly reproduces the tree's sums.
#pragma unroll
        for (int m = 8 / CPL; m >= 1; m >>= 1) {
#pragma unroll
            for (int s = 0; s < CPL; s++)
                sq[s] = sq[s] + __shfl_xor(sq[s], m);
            am = fmaxf(am, __shfl_xor(am, m));
        }
        float e = sq[0];
        if constexpr (CPL == 2)
            e = sq[0] + sq[1];
        if ((lane % (16 / CPL)) == 0) {
            sm.e[h][lane / (16 / CPL)] = e;
            sm.amax[h][lane / (16 / CPL)] = am;
        }
    }
    if constexpr (KF == KVQ_K_LLOYD4) {
        // code-pair table: byte (lo nibble a, hi nibble b) -> fp16 (cent[a], cent[b])
        sm.lut[tid] = pack_f16x2(p.codebook[tid & 15], p.codebook[tid >> 4]);
    }
    __syncthreads();

    // phase 2 (every thread, uniform): mask, then the query scale.
    uint32_t mask = (1u << NP) - 1u;
    if (p.keep > 0 && p.keep < NP) {
        float E[NP];
#pragma unroll
        for (int g = 0; g < NP; g++) {
            float acc = sm.e[0][g];
#pragma unroll
            for (int h = 1; h < G; h++)
                acc = acc + sm.e[h][g];
            E[g] = acc;
        }
        mask = 0;
#pragma unroll
        for (int g = 0; g < NP; g++) {
            int rank = 0;
#pragma unroll
            for (int o = 0; o < NP; o++)
                rank += (E[o] > E[g] || (E[o] == E[g] && o < g)) ? 1 : 0;
            if (rank < p.keep)
                mask |= 1u << g;
        }
    }
    mask = uniform(mask);
    if (split == 0 && tid == 0 && p.mask_out)
        p.mask_out[unit] = (uint8_t)mask;
    const float qscale = p.sm_log2e / (p.rotate ? (float)D : 1.0f);
    float amax = 0.0f;
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int g = 0; g < NP; g++)
            if (mask >> g & 1u)
                amax = fmaxf(amax, sm.amax[h][g]);
    amax *= qscale;
    // fp16 pair scale: largest scaled |q| lands in [2^12, 2^13)
    int ex = 0;
    (void)frexpf(amax, &ex);
    const float g2 = amax > 0.0f ? ldexpf(1.0f, 13 - ex) : 1.0f;
    __syncthreads();

    // phase 3: each wave writes its heads' scaled query, fp16 pairs and zero-term sums.
    for (int h = wave; h < G; h += kWavesPerBlock) {
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            const int c = lane * CPL + s;
            const bool kept = (mask >> (c / 16)) & 1u;
            sm.q[h][c] = kept ? sm.q[h][c] * qscale : 0.0f;
        }
    }
    __syncthreads();
    for (int h = wave; h < G; h += kWavesPerBlock) {
        if constexpr (KF == KVQ_K_LLOYD4) {
            // byte j of key word r holds channels (8r + 2j, 8r + 2j + 1)
            if (lane < KROWS * PPW) {
                const int r = lane / PPW, j = lane % PPW;
                const int ca = 8 * r + 2 * j;
                sm.qp[r][h][j] = pack_f16x2(sm.q[h][ca] * g2, sm.q[h][ca + 1] * g2);
            }
            if (lane == 0)
                sm.qsc[h] = 1.0f / g2;
        } else {
            // 16-bit integer query: q ~= qi * unit, |qi| <= 32639, written as 256*hi + lo
            // with signed bytes hi, lo.  Channel 0 is scored from its BF16 copy instead.
            float am = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < CPL; s2++) {
                const int c = lane * CPL + s2;
                if (!(p.ch0 && c == 0))
                    am = fmaxf(am, fabsf(sm.q[h][c]));
            }
            am = wave_max(am);
            const float unit_q = am > 0.0f ? am / 32639.0f : 1.0f;
            const float inv = 1.0f / unit_q;
            // key word r, spread register k: byte m holds channel r*(32/KB) + m*(KB==2 ? 4 : 2) + k
            if (lane < KROWS * C::NREG) {
                const int r = lane / C::NREG, k = lane % C::NREG;
                uint32_t hi = 0, lo = 0;
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    const int c = (KB == 2) ? 16 * r + 4 * m + k : 8 * r + 2 * m + k;
                    const float qv = (p.ch0 && c == 0) ? 0.0f : sm.q[h][c];
                    const int qi = (int)__builtin_rintf(qv * inv);
                    const int h8 = (qi + 128) >> 8;
                    const int l8 = qi - 256 * h8;
                    hi |= (uint32_t)(h8 & 0xFF) << (8 * m);
                    lo |= (uint32_t)(l8 & 0xFF) << (8 * m);
                }
                sm.qp[r][h][2 * k] = hi;
                sm.qp[r][h][2 * k + 1] = lo;
            }
            if (lane < NG) {
                float si = 0.0f;
                for (int c = 32 * lane; c < 32 * lane + 32; c++)
                    if (!(p.ch0 && c == 0))
                        si += __builtin_rintf(sm.q[h][c] * inv);
                sm.qz[h][lane] = si;
            }
            if (lane == 0) {
                sm.qsc[h] = unit_q;
                sm.q0[h] = (p.ch0 && (mask & 1u)) ? sm.q[h][0] * inv : 0.0f;
            }
        }
    }
    __syncthreads();
    float acc_to_logit[G];
#pragma unroll
    for (int h = 0; h < G; h++)
        acc_to_logit[h] = sm.qsc[h];

    // ------------------------------------------------------------------ state
    const int vs = lane % LPP;         // value slot: channels 16*vs .. 16*vs+15
    const int vgrp = vs >> 1;          // its scale group
    float acc[G][16];
    float zacc[G][NG];
    float lsum[G];
    float mrun[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        lsum[h] = 0.0f;
        mrun[h] = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 16; j++)
            acc[h][j] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; g++)
            zacc[h][g] = 0.0f;
    }
    const float chscale[2] = {5.9604644775390625e-08f, 9.5367431640625e-07f}; // 2^-24, 2^-20

    // ------------------------------------------------------------------ sink positions
    const int n_sink = p.n_sink < p.len ? p.n_sink : p.len;
    if (split == 0 && wave == 0 && n_sink > 0) {
        float sl[G];
        const bool valid = lane < n_sink;
        if (valid) {
            const uint16_t *sk = p.sink_k + ((size_t)unit * p.n_sink + lane) * D;
#pragma unroll
            for (int h = 0; h < G; h++)
                sl[h] = 0.0f;
            for (int c = 0; c < D; c += 2) {
                const uint32_t w = *reinterpret_cast<const uint32_t *>(sk + c);
                const float k0 = bf16_to_f32(w & 0xFFFFu), k1 = bf16_to_f32(w >> 16);
#pragma unroll
                for (int h = 0; h < G; h++)
                    sl[h] = fmaf(sm.q[h][c + 1], k1, fmaf(sm.q[h][c], k0, sl[h]));
            }
        }
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float x = valid ? sl[h] : -__builtin_inff();
            mrun[h] = uniformf(wave_max(x));
            const float pr = valid ? __builtin_amdgcn_exp2f(x - mrun[h]) : 0.0f;
            lsum[h] += pr;
            sm.sink_p[h][lane] = pr;
        }
        __builtin_amdgcn_wave_barrier();
        for (int t = lane / LPP; t < n_sink; t += PPI) {
            const uint16_t *sv = p.sink_v + ((size_t)unit * p.n_sink + t) * D + 16 * vs;
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const float v = bf16_to_f32(sv[j]) * chscale[j & 1];
#pragma unroll
                for (int h = 0; h < G; h++)
                    acc[h][j] = fmaf(sm.sink_p[h][t], v, acc[h][j]);
            }
        }
    }

    // ------------------------------------------------------------------ position tiles
    const int t_first = p.tile_begin + split * p.tiles_per_split;
    int t_last = t_first + p.tiles_per_split;
    if (t_last > p.tile_end)
        t_last = p.tile_end;
    const int q_lo = p.n_sink, q_hi = p.len; // quantized positions [q_lo, q_hi)
    const uint32_t *kc_base = p.k_codes + (size_t)unit * KROWS * cap;
    const uint32_t *ksz_base = p.k_sz + (size_t)unit * NG * cap;
    const uint32_t *vsz_base = p.v_sz + (size_t)unit * NG * cap;
    const uint32_t *vc_base = p.v_codes + (size_t)unit * (cap / 2) * WPP;

    for (int tile = t_first + wave; tile < t_last; tile += kWavesPerBlock) {
        const int t0 = tile * TILE;
        const int tl = t0 + lane * TPL;
        // ---- loads
        uint4 kc[KROWS];
#pragma unroll
        for (int r = 0; r < KROWS; r++)
            if (mask >> (r / C::RPP) & 1u)
                kc[r] = *reinterpret_cast<const uint4 *>(kc_base + (size_t)r * cap + tl);
        uint4 ksz[NG];
        uint2 knorm;
        if constexpr (KF != KVQ_K_LLOYD4) {
#pragma unroll
            for (int g = 0; g < NG; g++)
                if (mask >> (2 * g) & 3u)
                    ksz[g] = *reinterpret_cast<const uint4 *>(ksz_base + (size_t)g * cap + tl);
        } else {
            knorm = *reinterpret_cast<const uint2 *>(p.k_norm + (size_t)unit * cap + tl);
        }
        uint2 k0w = make_uint2(0, 0);
        if (KF != KVQ_K_LLOYD4 && p.ch0 && (mask & 1u))
            k0w = *reinterpret_cast<const uint2 *>(p.k_ch0 + (size_t)unit * cap + tl);
        uint4 vsz[NG];
#pragma unroll
        for (int g = 0; g < NG; g++)
            vsz[g] = *reinterpret_cast<const uint4 *>(vsz_base + (size_t)g * cap + tl);
        uint4 vw[VIT];
#pragma unroll
        for (int it = 0; it < VIT; it++) {
            const size_t pair = (size_t)(t0 / 2 + it * PPI + lane / LPP);
            vw[it] = *reinterpret_cast<const uint4 *>(vc_base + pair * WPP + 4 * vs);
        }

        // ---- scores (accumulator units; log2 logit = lg * acc_to_logit)
        float lg[TPL][G];
#pragma unroll
        for (int i = 0; i < TPL; i++)
#pragma unroll
            for (int h = 0; h < G; h++)
                lg[i][h] = 0.0f;
        if constexpr (KF != KVQ_K_LLOYD4) {
            constexpr int NREG = C::NREG;
#pragma unroll
            for (int g = 0; g < NG; g++) {
                if (!(mask >> (2 * g) & 3u))
                    continue;
                int dh[TPL][G], dl[TPL][G];
#pragma unroll
                for (int i = 0; i < TPL; i++)
#pragma unroll
                    for (int h = 0; h < G; h++) {
                        dh[i][h] = 0;
                        dl[i][h] = 0;
                    }
#pragma unroll
                for (int rr = 0; rr < KROWS / NG; rr++) {
                    const int r = g * (KROWS / NG) + rr;
                    if (!(mask >> (r / C::RPP) & 1u))
                        continue;
                    uint32_t qh[G][NREG], ql[G][NREG];
#pragma unroll
                    for (int h = 0; h < G; h++)
#pragma unroll
                        for (int k = 0; k < NREG; k++) {
                            qh[h][k] = uniform(sm.qp[r][h][2 * k]);
                            ql[h][k] = uniform(sm.qp[r][h][2 * k + 1]);
                        }
#pragma unroll
                    for (int i = 0; i < TPL; i++) {
                        const uint32_t x = (i == 0) ? kc[r].x : (i == 1) ? kc[r].y : (i == 2) ? kc[r].z : kc[r].w;
                        uint32_t bsp[NREG];
                        if constexpr (KB == 2) {
                            bsp[0] = x & 0x03030303u;
                            bsp[1] = (x >> 2) & 0x03030303u;
                            bsp[2] = (x >> 4) & 0x03030303u;
                            bsp[3] = (x >> 6) & 0x03030303u;
                        } else {
                            bsp[0] = x & 0x0F0F0F0Fu;
                            bsp[1] = (x >> 4) & 0x0F0F0F0Fu;
                        }
#pragma unroll
                        for (int h = 0; h < G; h++)
#pragma unroll
                            for (int k = 0; k < NREG; k++) {
                                dh[i][h] = __builtin_amdgcn_sdot4((int)qh[h][k], (int)bsp[k], dh[i][h], false);
                                dl[i][h] = __builtin_amdgcn_sdot4((int)ql[h][k], (int)bsp[k], dl[i][h], false);
                            }
                    }
                }
#pragma unroll
                for (int i = 0; i < TPL; i++) {
                    const uint32_t szw = (i == 0) ? ksz[g].x : (i == 1) ? ksz[g].y : (i == 2) ? ksz[g].z : ksz[g].w;
                    const float s = lo_f16(szw), z = hi_f16(szw);
#pragma unroll
                    for (int h = 0; h < G; h++) {
                        const float dsum = (float)(dh[i][h] * 256 + dl[i][h]);
                        lg[i][h] = fmaf(z, sm.qz[h][g], fmaf(s, dsum, lg[i][h]));
                    }
                }
            }
            if (p.ch0 && (mask & 1u)) {
#pragma unroll
                for (int i = 0; i < TPL; i++) {
                    const uint32_t w = (i < 2) ? k0w.x : k0w.y;
                    const float k0 = bf16_to_f32((i & 1) ? (w >> 16) : (w & 0xFFFFu));
#pragma unroll
                    for (int h = 0; h < G; h++)
                        lg[i][h] = fmaf(k0, sm.q0[h], lg[i][h]);
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < KROWS; r++) {
                if (!(mask >> (r / C::RPP) & 1u))
                    continue;
                uint32_t qp[G][PPW];
#pragma unroll
                for (int h = 0; h < G; h++)
#pragma unroll
                    for (int j = 0; j < PPW; j++)
                        qp[h][j] = uniform(sm.qp[r][h][j]);
#pragma unroll
                for (int i = 0; i < TPL; i++) {
                    const uint32_t x = (i == 0) ? kc[r].x : (i == 1) ? kc[r].y : (i == 2) ? kc[r].z : kc[r].w;
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const uint32_t pr = sm.lut[(x >> (8 * j)) & 0xFFu];
#pragma unroll
                        for (int h = 0; h < G; h++)
                            lg[i][h] = dot2(pr, qp[h][j], lg[i][h]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < TPL; i++) {
                const uint32_t w = (i < 2) ? knorm.x : knorm.y;
                const float rho = f16_to_f32((i & 1) ? (w >> 16) : (w & 0xFFFFu));
#pragma unroll
                for (int h = 0; h < G; h++)
                    lg[i][h] *= rho;
            }
        }

        // ---- mask positions outside [q_lo, q_hi) (their slots may hold anything)
        const bool full = (t0 >= q_lo) && (t0 + TILE <= q_hi);
        float vs_s[TPL][NG], vs_z[TPL][NG];
#pragma unroll
        for (int i = 0; i < TPL; i++)
#pragma unroll
            for (int g = 0; g < NG; g++) {
                const uint32_t szw = (i == 0) ? vsz[g].x : (i == 1) ? vsz[g].y : (i == 2) ? vsz[g].z : vsz[g].w;
                vs_s[i][g] = lo_f16(szw);
                vs_z[i][g] = hi_f16(szw);
            }
        if (!full) {
#pragma unroll
            for (int i = 0; i < TPL; i++) {
                const int t = tl + i;
                if (t < q_lo || t >= q_hi) {
#pragma unroll
                    for (int h = 0; h < G; h++)
                        lg[i][h] = -__builtin_inff();
#pragma unroll
                    for (int g = 0; g < NG; g++) {
                        vs_s[i][g] = 0.0f;
                        vs_z[i][g] = 0.0f;
                    }
                }
            }
        }

        // ---- online softmax (log2 units)
        float mnew[G];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < G; h++) {
            float mt = lg[0][h];
#pragma unroll
            for (int i = 1; i < TPL; i++)
                mt = fmaxf(mt, lg[i][h]);
            mt = uniformf(wave_max(mt)) * acc_to_logit[h];
            mnew[h] = fmaxf(mrun[h], mt);
            grow |= mnew[h] > mrun[h];
        }
        if (grow) {
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float alpha = __builtin_amdgcn_exp2f(mrun[h] - mnew[h]);
                mrun[h] = mnew[h];
                lsum[h] *= alpha;
#pragma unroll
                for (int j = 0; j < 16; j++)
                    acc[h][j] *= alpha;
#pragma unroll
                for (int g = 0; g < NG; g++)
                    zacc[h][g] *= alpha;
            }
        }
        float pw[TPL][G];
#pragma unroll
        for (int i = 0; i < TPL; i++)
#pragma unroll
            for (int h = 0; h < G; h++) {
                pw[i][h] = __builtin_amdgcn_exp2f(fmaf(lg[i][h], acc_to_logit[h], -mrun[h]));
                lsum[h] += pw[i][h];
            }
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int g = 0; g < NG; g++)
#pragma unroll
                for (int i = 0; i < TPL; i++)
                    zacc[h][g] = fmaf(pw[i][h], vs_z[i][g], zacc[h][g]);
        // weights p*s as fp16 pairs over positions (2m, 2m+1) -> LDS
#pragma unroll
        for (int ip = 0; ip < TPL / 2; ip++) {
            uint32_t *dst = &sm.u.w[wave][lane * (TPL / 2) + ip][0];
#pragma unroll
            for (int g = 0; g < NG; g++)
#pragma unroll
                for (int h = 0; h < G; h++)
                    dst[g * G + h] = pack_f16x2(pw[2 * ip][h] * vs_s[2 * ip][g], pw[2 * ip + 1][h] * vs_s[2 * ip + 1][g]);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

        // ---- values
#pragma unroll
        for (int it = 0; it < VIT; it++) {
            const int pl = it * PPI + lane / LPP;
            uint32_t wv[G];
#pragma unroll
            for (int h = 0; h < G; h++)
                wv[h] = sm.u.w[wave][pl][vgrp * G + h];
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const uint32_t x = (q4 == 0) ? vw[it].x : (q4 == 1) ? vw[it].y : (q4 == 2) ? vw[it].z : vw[it].w;
                const uint32_t y = x >> 8;
                const uint32_t c0 = x & 0x000F000Fu, c1 = x & 0x00F000F0u;
                const uint32_t c2 = y & 0x000F000Fu, c3 = y & 0x00F000F0u;
#pragma unroll
                for (int h = 0; h < G; h++) {
                    acc[h][4 * q4 + 0] = dot2(c0, wv[h], acc[h][4 * q4 + 0]);
                    acc[h][4 * q4 + 1] = dot2(c1, wv[h], acc[h][4 * q4 + 1]);
                    acc[h][4 * q4 + 2] = dot2(c2, wv[h], acc[h][4 * q4 + 2]);
                    acc[h][4 * q4 + 3] = dot2(c3, wv[h], acc[h][4 * q4 + 3]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }

    // ------------------------------------------------------------------ wave reduction
#pragma unroll
    for (int h = 0; h < G; h++) {
        lsum[h] = wave_sum(lsum[h]);
#pragma unroll
        for (int g = 0; g < NG; g++)
            zacc[h][g] = wave_sum(zacc[h][g]);
#pragma unroll
        for (int j = 0; j < 16; j++)
#pragma unroll
            for (int m = LPP; m < 64; m <<= 1)
                acc[h][j] += __shfl_xor(acc[h][j], m);
    }
    __syncthreads(); // the weight buffer is reused for the merge below
    if (lane < LPP) {
#pragma unroll
        for (int h = 0; h < G; h++) {
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const float sc = (j & 1) ? 1048576.0f : 16777216.0f; // undo 2^-20 / 2^-24
                sm.u.merge[wave][h][2 + 16 * lane + j] = acc[h][j] * sc + zacc[h][(16 * lane + j) / 32];
            }
            if (lane == 0) {
                sm.u.merge[wave][h][0] = mrun[h];
                sm.u.merge[wave][h][1] = lsum[h];
            }
        }
    }
    __syncthreads();

    // ------------------------------------------------------------------ workgroup merge
    // thread (h, c): combine the 4 waves' states; write this split's partial or the output.
    const bool single = (p.n_split == 1);
    for (int idx = tid; idx < G * (D + 2); idx += kBlock) {
        const int h = idx / (D + 2);
        const int c = idx % (D + 2);
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; w++)
            M = fmaxf(M, sm.u.merge[w][h][0]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; w++) {
            const float mw = sm.u.merge[w][h][0];
            const float f = (mw == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            L = fmaf(sm.u.merge[w][h][1], f, L);
            if (c >= 2)
                O = fmaf(sm.u.merge[w][h][c], f, O);
        }
        if (single) {
            if (c >= 2) {
                const size_t oi = ((size_t)b * n_q_heads + (size_t)kvh * G + h) * D + (c - 2);
                p.out[oi] = L > 0.0f ? O / L : 0.0f;
            }
        } else {
            float *part = p.part + (((size_t)unit * p.n_split + split) * G + h) * (D + 2);
            part[c] = (c == 0) ? M : (c == 1) ? L : O;
        }
    }
    if (single)
        return;

    // ------------------------------------------------------------------ split merge
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t ticket = atomicAdd(p.counters + unit, 1u);
        sm.last = (ticket == (uint32_t)(p.n_split - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!sm.last)
        return;
    __threadfence();
    const float *pbase = p.part + (size_t)unit * p.n_split * G * (D + 2);
    for (int idx = tid; idx < G * D; idx += kBlock) {
        const int h = idx / D;
        const int c = idx % D;
        float M = -__builtin_inff();
        for (int s = 0; s < p.n_split; s++)
            M = fmaxf(M, __builtin_nontemporal_load(pbase + ((size_t)s * G + h) * (D + 2)));
        float L = 0.0f, O = 0.0f;
        for (int s = 0; s < p.n_split; s++) {
            const float *ps = pbase + ((size_t)s * G + h) * (D + 2);
            const float ms = __builtin_nontemporal_load(ps);
            const float f = (ms == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
            L = fmaf(__builtin_nontemporal_load(ps + 1), f, L);
            O = fmaf(__builtin_nontemporal_load(ps + 2 + c), f, O);
        }
        const size_t oi = ((size_t)b * n_q_heads + (size_t)kvh * G + h) * D + c;
        p.out[oi] = L > 0.0f ? O / L : 0.0f;
    }
    if (tid == 0)
        p.counters[unit] = 0u; // ready for the next call on this stream
}

template <int D, int G, int KF>
hipError_t launch_one(int units, const DecodeParams &p, hipStream_t s)
{
    dim3 grid((unsigned)p.n_split, (unsigned)units), block(kBlock);
    hipLaunchKernelGGL((decode_kernel<D, G, KF>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_kf(int kfmt, int units, const DecodeParams &p, hipStream_t s)
{
    switch (kfmt) {
    case KVQ_K_ASYM2: return launch_one<D, G, KVQ_K_ASYM2>(units, p, s);
    case KVQ_K_ASYM4: return launch_one<D, G, KVQ_K_ASYM4>(units, p, s);
    default: return launch_one<D, G, KVQ_K_LLOYD4>(units, p, s);
    }
}

template <int D>
hipError_t launch_g(int group, int kfmt, int units, const DecodeParams &p, hipStream_t s)
{
    switch (group) {
    case 1: return launch_kf<D, 1>(kfmt, units, p, s);
    case 2: return launch_kf<D, 2>(kfmt, units, p, s);
    case 4: return launch_kf<D, 4>(kfmt, units, p, s);
    default: return launch_kf<D, 8>(kfmt, units, p, s);
    }
}

} // namespace

hipError_t launch_decode(int head_dim, int group, int kfmt, int units, const DecodeParams &p,
                         hipStream_t s)
{
    if (head_dim == 128)
        return launch_g<128>(group, kfmt, units, p, s);
    return launch_g<64>(group, kfmt, units, p, s);
}

} // namespace kvq
