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
//     merged across splits by a small second kernel (no device-wide fences);
//   * values from INT4 codes: o = sum_t p_t s_{t,g} code_{t,c} + sum_t p_t z_{t,g}.
//
// MI355X mapping (one workgroup = one wave = one context split of one unit; the host sizes
// the splits so every SIMD slot the kernel's register use allows holds a wave):
//   * score phase, lane per position: each lane scores 2 consecutive positions; a key row
//     is one dwordx2 load per lane (64 lanes read 512 B contiguous).  Asymmetric codes are
//     spread into bytes by shift+mask and multiplied with v_dot4_i32_i8 against the query
//     held as a 16-bit integer in two signed-byte planes: exact int32 sums, and the
//     zero-point term uses the same integer query, so code and zero terms together equal
//     q_int . k^ with no cancellation between them (heavy-tailed keys make the group zero
//     large).  The planes of one (row, head) come from LDS as a broadcast read straight into
//     VGPR operands.  Lloyd-Max codes go through an LDS table of fp16 centroid pairs and
//     v_dot2_f32_f16 against fp16 query pairs.
//   * softmax: a running maximum per head; a wave-wide DPP reduction and a rescale happen
//     only when a tile holds a logit above it (rare after the first tiles).
//   * value phase, lane per 8 channels: v_dot2_f32_f16 over position pairs (value words
//     interleave two positions); a 4-bit code masked into the low mantissa bits of a half
//     is the subnormal integer code * 2^-24 (or * 2^-20), so no conversion is needed.  The
//     fp16 weights p*s of each position pair come from LDS (conflict-free layout).
//   * the next tile's key-side words are loaded before the value phase of the current one.
//   * no MFMA: this is a bandwidth-bound scan.
#include <atomic>

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
    static constexpr int QW = (KF == KVQ_K_LLOYD4) ? 4 : 2 * NREG; // query words per (row, head)
    static constexpr int NG = D / 32;              // scale groups
    static constexpr int NP = D / 16;              // prune groups
    static constexpr int RPP = 16 * KB / 32;       // key rows per prune group
    static constexpr int TPL = 2;                  // positions per lane in the score phase
    static constexpr int TILE = 64 * TPL;
    static constexpr int PAIRS = TILE / 2;
    static constexpr int WPP = D / 4;              // value words per position pair
    static constexpr int VW = 2;                   // value words per lane per iteration
    static constexpr int LPP = WPP / VW;           // value lanes per pair
    static constexpr int PPI = 64 / LPP;           // pairs per value iteration
    static constexpr int VIT = PAIRS / PPI;        // value iterations per tile
    static constexpr int CPL = D / 64;             // channels per lane in the prologue
    static constexpr int WROW = PAIRS + 1;         // padded LDS weight row (conflict-free)
    static_assert(TILE == kTile, "host and device tile must agree");
};

template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_max_step(float x)
{
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROWMASK, 0xF, false);
    return fmaxf(x, __int_as_float(o));
}

// max over the wave, result in every lane (DPP row shifts, then row broadcasts to lane 63)
__device__ __forceinline__ float wave_max_dpp(float v)
{
    v = dpp_max_step<0x111, 0xF>(v); // row_shr:1
    v = dpp_max_step<0x112, 0xF>(v); // row_shr:2
    v = dpp_max_step<0x114, 0xF>(v); // row_shr:4
    v = dpp_max_step<0x118, 0xF>(v); // row_shr:8
    v = dpp_max_step<0x142, 0xA>(v); // row_bcast:15
    v = dpp_max_step<0x143, 0xC>(v); // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

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
    uint4 qp[C::KROWS][G][C::QW / 4];               // per (key row, head): int8 hi/lo query
                                                    // planes (asym) or fp16 pairs (Lloyd-Max)
    float qz[G][C::NG];                             // zero-term integer query sums
    float q0[G];                                    // channel-0 coefficient (integer units)
    float qsc[G];                                   // accumulator unit in log2-logit units
    uint32_t lut[KF == KVQ_K_LLOYD4 ? 256 : 1];     // Lloyd-Max code-pair table (fp16x2)
    float sink_p[G][kMaxSink];
    uint32_t w[C::NG * G][C::WROW];                 // fp16 weight pairs of the current tile
};

// Key-side words of one tile for this lane (TPL = 2 positions).
template <int D, int G, int KF>
struct KTile {
    using C = Cfg<D, G, KF>;
    uint2 kc[C::KROWS];
    uint2 ksz[C::NG];
    uint2 vsz[C::NG];
    uint32_t kx; // channel-0 bf16 pair (asym + protection) or rho fp16 pair (Lloyd-Max)
};

template <int D, int G, int KF>
__device__ __forceinline__ void load_ktile(KTile<D, G, KF> &k, const DecodeParams &p, int unit, int tl,
                                           uint32_t mask)
{
    using C = Cfg<D, G, KF>;
    const size_t cap = (size_t)p.cap;
    const uint32_t *kc_base = p.k_codes + (size_t)unit * C::KROWS * cap + tl;
#pragma unroll
    for (int r = 0; r < C::KROWS; r++)
        if (mask >> (r / C::RPP) & 1u)
            k.kc[r] = *reinterpret_cast<const uint2 *>(kc_base + (size_t)r * cap);
    if constexpr (KF != KVQ_K_LLOYD4) {
        const uint32_t *ksz_base = p.k_sz + (size_t)unit * C::NG * cap + tl;
#pragma unroll
        for (int g = 0; g < C::NG; g++)
            if (mask >> (2 * g) & 3u)
                k.ksz[g] = *reinterpret_cast<const uint2 *>(ksz_base + (size_t)g * cap);
        k.kx = 0;
        if (p.ch0 && (mask & 1u))
            k.kx = *reinterpret_cast<const uint32_t *>(p.k_ch0 + (size_t)unit * cap + tl);
    } else {
        k.kx = *reinterpret_cast<const uint32_t *>(p.k_norm + (size_t)unit * cap + tl);
    }
    const uint32_t *vsz_base = p.v_sz + (size_t)unit * C::NG * cap + tl;
#pragma unroll
    for (int g = 0; g < C::NG; g++)
        k.vsz[g] = *reinterpret_cast<const uint2 *>(vsz_base + (size_t)g * cap);
}

// Asymmetric-key logits of this lane's TPL positions in accumulator units:
//   lg = sum_g s_g * (q_int . code)_g + z_g * sum_{c in g} q_int_c  (+ k0 * q0)
// ALL: every 16-channel row is kept (no pruning), so the row tests fold away.
// Per (group, head, position) one int32 sum collects the hi-plane products, is shifted
// by 8, then collects the lo-plane products: sum = 256 * hi.code + lo.code = q_int.code.
template <int D, int G, int KF, bool ALL>
__device__ __forceinline__ void score_asym(const KTile<D, G, KF> &cur, const Smem<D, G, KF> &sm, uint32_t mask,
                                           int ch0, float (&lg)[Cfg<D, G, KF>::TPL][G])
{
    using C = Cfg<D, G, KF>;
    constexpr int KB = C::KB, KROWS = C::KROWS, NG = C::NG, TPL = C::TPL, NREG = C::NREG, QW = C::QW;
    constexpr int RPG = KROWS / NG; // key rows per scale group
#pragma unroll
    for (int g = 0; g < NG; g++) {
        if (!ALL && !(mask >> (2 * g) & 3u))
            continue;
        uint32_t bsp[RPG][TPL][NREG];
#pragma unroll
        for (int rr = 0; rr < RPG; rr++) {
            const int r = g * RPG + rr;
#pragma unroll
            for (int i = 0; i < TPL; i++) {
                const uint32_t x = i == 0 ? cur.kc[r].x : cur.kc[r].y;
                if constexpr (KB == 2) {
                    bsp[rr][i][0] = x & 0x03030303u;
                    bsp[rr][i][1] = (x >> 2) & 0x03030303u;
                    bsp[rr][i][2] = (x >> 4) & 0x03030303u;
                    bsp[rr][i][3] = (x >> 6) & 0x03030303u;
                } else {
                    bsp[rr][i][0] = x & 0x0F0F0F0Fu;
                    bsp[rr][i][1] = (x >> 4) & 0x0F0F0F0Fu;
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; h++) {
            int acc[TPL];
#pragma unroll
            for (int i = 0; i < TPL; i++)
                acc[i] = 0;
#pragma unroll
            for (int plane = 0; plane < 2; plane++) {
                if (plane == 1) {
#pragma unroll
                    for (int i = 0; i < TPL; i++)
                        acc[i] <<= 8;
                }
#pragma unroll
                for (int rr = 0; rr < RPG; rr++) {
                    const int r = g * RPG + rr;
                    if (!ALL && !(mask >> (r / C::RPP) & 1u))
                        continue;
                    // broadcast LDS read of this (row, head)'s plane words into VGPRs
                    const uint4 t4 = sm.qp[r][h][(plane * NREG) / 4];
                    uint32_t qw[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                    for (int i = 0; i < TPL; i++)
#pragma unroll
                        for (int k = 0; k < NREG; k++)
                            acc[i] = __builtin_amdgcn_sdot4((int)qw[(plane * NREG) % 4 + k], (int)bsp[rr][i][k], acc[i], false);
                }
            }
#pragma unroll
            for (int i = 0; i < TPL; i++) {
                const uint32_t szw = i == 0 ? cur.ksz[g].x : cur.ksz[g].y;
                lg[i][h] = fmaf(hi_f16(szw), sm.qz[h][g], fmaf(lo_f16(szw), (float)acc[i], lg[i][h]));
            }
        }
    }
    if (ch0 && (mask & 1u)) {
#pragma unroll
        for (int i = 0; i < TPL; i++) {
            const float k0 = bf16_to_f32(i == 0 ? (cur.kx & 0xFFFFu) : (cur.kx >> 16));
#pragma unroll
            for (int h = 0; h < G; h++)
                lg[i][h] = fmaf(k0, sm.q0[h], lg[i][h]);
        }
    }
}

template <int D, int G, int KF>
__global__ __launch_bounds__(kWave) void decode_kernel(DecodeParams p)
{
    using C = Cfg<D, G, KF>;
    constexpr int KB = C::KB, KROWS = C::KROWS, PPW = C::PPW, NG = C::NG, NP = C::NP;
    constexpr int TPL = C::TPL, TILE = C::TILE, WPP = C::WPP, LPP = C::LPP, PPI = C::PPI;
    constexpr int VIT = C::VIT, CPL = C::CPL, QW = C::QW, VW = C::VW;
    __shared__ Smem<D, G, KF> sm;

    const int lane = threadIdx.x;
    const int split = blockIdx.x;
    const int unit = blockIdx.y;
    const int b = unit / p.n_kv_heads;
    const int kvh = unit % p.n_kv_heads;
    const size_t cap = (size_t)p.cap;
    const int n_q_heads = p.n_kv_heads * G;

    // ------------------------------------------------------------------ prologue
    // phase 1: for each head: fp32 query in stored coordinates (FWHT when keys are
    // rotated), 16-channel group energies and max |q|.
    for (int h = 0; h < G; h++) {
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
        for (int e = lane; e < 256; e += kWave)
            sm.lut[e] = pack_f16x2(p.codebook[e & 15], p.codebook[e >> 4]);
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
    if (split == 0 && lane == 0 && p.mask_out)
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
    // Lloyd-Max fp16 pair scale: the largest scaled |q| lands in [2^12, 2^13)
    int ex = 0;
    (void)frexpf(amax, &ex);
    const float g2 = amax > 0.0f ? ldexpf(1.0f, 13 - ex) : 1.0f;
    __syncthreads();

    // phase 3: scaled query, query operands and zero-term sums of every head.
    for (int h = 0; h < G; h++) {
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            const int c = lane * CPL + s;
            const bool kept = (mask >> (c / 16)) & 1u;
            sm.q[h][c] = kept ? sm.q[h][c] * qscale : 0.0f;
        }
    }
    __syncthreads();
    for (int h = 0; h < G; h++) {
        uint32_t *qpw = reinterpret_cast<uint32_t *>(&sm.qp[0][0][0]);
        if constexpr (KF == KVQ_K_LLOYD4) {
            // byte j of key word r holds channels (8r + 2j, 8r + 2j + 1)
            if (lane < KROWS * PPW) {
                const int r = lane / PPW, j = lane % PPW;
                const int ca = 8 * r + 2 * j;
                qpw[(r * G + h) * QW + j] = pack_f16x2(sm.q[h][ca] * g2, sm.q[h][ca + 1] * g2);
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
            am = wave_max_dpp(am);
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
                // word layout per (row, head): hi planes of regs 0..NREG-1, then lo planes
                qpw[(r * G + h) * QW + k] = hi;
                qpw[(r * G + h) * QW + C::NREG + k] = lo;
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
    const bool all_rows = mask == (1u << NP) - 1u;

    // ------------------------------------------------------------------ state
    const int vs = lane % LPP;         // value slot: channels 8*vs .. 8*vs+7
    const int vgrp = vs / 4;           // its scale group
    float acc[G][8];
    float zacc[G][NG];
    float lsum[G];
    float mrun[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        lsum[h] = 0.0f;
        mrun[h] = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 8; j++)
            acc[h][j] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; g++)
            zacc[h][g] = 0.0f;
    }
    const float chscale[2] = {5.9604644775390625e-08f, 9.5367431640625e-07f}; // 2^-24, 2^-20

    // ------------------------------------------------------------------ sink positions
    const int n_sink = p.n_sink < p.len ? p.n_sink : p.len;
    if (split == 0 && n_sink > 0) {
        float sl[G];
        const bool valid = lane < n_sink;
#pragma unroll
        for (int h = 0; h < G; h++)
            sl[h] = 0.0f;
        if (valid) {
            const uint16_t *sk = p.sink_k + ((size_t)unit * p.n_sink + lane) * D;
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
            mrun[h] = wave_max_dpp(x);
            const float pr = valid ? __builtin_amdgcn_exp2f(x - mrun[h]) : 0.0f;
            lsum[h] += pr;
            sm.sink_p[h][lane] = pr;
        }
        __builtin_amdgcn_wave_barrier();
        for (int t = lane / LPP; t < n_sink; t += PPI) {
            const uint16_t *sv = p.sink_v + ((size_t)unit * p.n_sink + t) * D + 8 * vs;
#pragma unroll
            for (int j = 0; j < 8; j++) {
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
    const uint32_t *vc_base = p.v_codes + (size_t)unit * (cap / 2) * WPP + VW * vs;
    uint32_t(&wl)[NG * G][C::WROW] = sm.w;

    KTile<D, G, KF> cur;
    int tile = t_first;
    if (tile < t_last)
        load_ktile<D, G, KF>(cur, p, unit, tile * TILE + lane * TPL, mask);
    for (; tile < t_last; tile++) {
        const int t0 = tile * TILE;
        const int tl = t0 + lane * TPL;
        // keep the per-(row, head) query reads inside the loop: hoisting all of them out
        // would pin KROWS*G*QW registers for the whole loop
        asm volatile("" ::: "memory");

        // ---- scores (accumulator units; log2 logit = lg * acc_to_logit[h])
        float lg[TPL][G];
#pragma unroll
        for (int i = 0; i < TPL; i++)
#pragma unroll
            for (int h = 0; h < G; h++)
                lg[i][h] = 0.0f;
        if constexpr (KF != KVQ_K_LLOYD4) {
            if (all_rows)
                score_asym<D, G, KF, true>(cur, sm, mask, p.ch0, lg);
            else
                score_asym<D, G, KF, false>(cur, sm, mask, p.ch0, lg);
        } else {
#pragma unroll
            for (int r = 0; r < KROWS; r++) {
                if (!(mask >> (r / C::RPP) & 1u))
                    continue;
                uint32_t pr[TPL][4];
#pragma unroll
                for (int i = 0; i < TPL; i++) {
                    const uint32_t x = i == 0 ? cur.kc[r].x : cur.kc[r].y;
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        pr[i][j] = sm.lut[(x >> (8 * j)) & 0xFFu];
                }
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const uint4 qv = sm.qp[r][h][0];
                    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                    for (int i = 0; i < TPL; i++)
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            lg[i][h] = dot2(pr[i][j], qw[j], lg[i][h]);
                }
            }
#pragma unroll
            for (int i = 0; i < TPL; i++) {
                const float rho = f16_to_f32(i == 0 ? (cur.kx & 0xFFFFu) : (cur.kx >> 16));
#pragma unroll
                for (int h = 0; h < G; h++)
                    lg[i][h] *= rho;
            }
        }

        // ---- value scale/zero of this lane's positions; mask positions outside
        // [q_lo, q_hi) (their slots may hold anything)
        float vs_s[TPL][NG], vs_z[TPL][NG];
#pragma unroll
        for (int i = 0; i < TPL; i++)
#pragma unroll
            for (int g = 0; g < NG; g++) {
                const uint32_t szw = i == 0 ? cur.vsz[g].x : cur.vsz[g].y;
                vs_s[i][g] = lo_f16(szw);
                vs_z[i][g] = hi_f16(szw);
            }
        const bool full = (t0 >= q_lo) && (t0 + TILE <= q_hi);
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

        // ---- next tile's key-side words, into the registers this tile no longer needs:
        // in flight during the rest of this tile
        if (tile + 1 < t_last)
            load_ktile<D, G, KF>(cur, p, unit, (tile + 1) * TILE + lane * TPL, mask);

        // ---- online softmax (log2 units); wave-wide max only when some logit exceeds
        // the running maximum
        float lmax[G];
        bool above = false;
#pragma unroll
        for (int h = 0; h < G; h++) {
            float mt = lg[0][h];
#pragma unroll
            for (int i = 1; i < TPL; i++)
                mt = fmaxf(mt, lg[i][h]);
            lmax[h] = mt * acc_to_logit[h];
            above |= lmax[h] > mrun[h];
        }
        if (__any(above)) {
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float mnew = fmaxf(mrun[h], wave_max_dpp(lmax[h]));
                const float alpha = __builtin_amdgcn_exp2f(mrun[h] - mnew);
                mrun[h] = mnew;
                lsum[h] *= alpha;
#pragma unroll
                for (int j = 0; j < 8; j++)
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
        // weights p*s as fp16 pairs over positions (2m, 2m+1) -> LDS row (g, h), column pair
#pragma unroll
        for (int g = 0; g < NG; g++)
#pragma unroll
            for (int h = 0; h < G; h++)
                wl[g * G + h][lane] = pack_f16x2(pw[0][h] * vs_s[0][g], pw[1][h] * vs_s[1][g]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- values: lane owns channels 8*vs .. 8*vs+7 of one pair per iteration
        const uint32_t *vrow = vc_base + (size_t)(t0 / 2 + lane / LPP) * WPP;
#pragma unroll
        for (int it = 0; it < VIT; it++) {
            const uint2 vv = *reinterpret_cast<const uint2 *>(vrow + (size_t)it * PPI * WPP);
            const int pl = it * PPI + lane / LPP;
            uint32_t wv[G];
#pragma unroll
            for (int h = 0; h < G; h++)
                wv[h] = wl[vgrp * G + h][pl];
#pragma unroll
            for (int q2 = 0; q2 < 2; q2++) {
                const uint32_t x = q2 == 0 ? vv.x : vv.y;
                const uint32_t y = x >> 8;
                const uint32_t c0 = x & 0x000F000Fu, c1 = x & 0x00F000F0u;
                const uint32_t c2 = y & 0x000F000Fu, c3 = y & 0x00F000F0u;
#pragma unroll
                for (int h = 0; h < G; h++) {
                    acc[h][4 * q2 + 0] = dot2(c0, wv[h], acc[h][4 * q2 + 0]);
                    acc[h][4 * q2 + 1] = dot2(c1, wv[h], acc[h][4 * q2 + 1]);
                    acc[h][4 * q2 + 2] = dot2(c2, wv[h], acc[h][4 * q2 + 2]);
                    acc[h][4 * q2 + 3] = dot2(c3, wv[h], acc[h][4 * q2 + 3]);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ------------------------------------------------------------------ wave reduction
#pragma unroll
    for (int h = 0; h < G; h++) {
        lsum[h] = wave_sum(lsum[h]);
#pragma unroll
        for (int g = 0; g < NG; g++)
            zacc[h][g] = wave_sum(zacc[h][g]);
#pragma unroll
        for (int j = 0; j < 8; j++)
#pragma unroll
            for (int m = LPP; m < 64; m <<= 1)
                acc[h][j] += __shfl_xor(acc[h][j], m);
    }
    // lanes 0..LPP-1 hold channels 8*lane .. 8*lane+7: the split's partial (m, l, o), or the
    // normalised output when the whole context is one split
    if (lane < LPP) {
        const bool single = (p.n_split == 1);
#pragma unroll
        for (int h = 0; h < G; h++) {
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float sc = (j & 1) ? 1048576.0f : 16777216.0f; // undo 2^-20 / 2^-24
                o[j] = acc[h][j] * sc + zacc[h][(8 * lane + j) / 32];
            }
            if (single) {
                const float inv = lsum[h] > 0.0f ? 1.0f / lsum[h] : 0.0f;
                float4 *dst = reinterpret_cast<float4 *>(p.out + ((size_t)b * n_q_heads + (size_t)kvh * G + h) * D + 8 * lane);
                dst[0] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
                dst[1] = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
            } else {
                float *part = p.part + (((size_t)unit * p.n_split + split) * G + h) * (D + 2);
                if (lane == 0) {
                    part[0] = mrun[h];
                    part[1] = lsum[h];
                }
#pragma unroll
                for (int j = 0; j < 8; j++)
                    part[2 + 8 * lane + j] = o[j];
            }
        }
    }
}

// Split merge: one thread per (sequence, query head, channel) combines the per-split
// (m, l, o) partials -- one global softmax over all positions (Dual-QK sec. 3.4).
template <int D, int G>
__global__ __launch_bounds__(D) void merge_kernel(DecodeParams p)
{
    const int c = threadIdx.x;
    const int h = blockIdx.x;
    const int unit = blockIdx.y;
    const int b = unit / p.n_kv_heads;
    const int kvh = unit % p.n_kv_heads;
    const float *pbase = p.part + ((size_t)unit * p.n_split * G + h) * (D + 2);
    const size_t stride = (size_t)G * (D + 2);
    float M = -__builtin_inff();
    for (int s = 0; s < p.n_split; s++)
        M = fmaxf(M, pbase[s * stride]);
    float L = 0.0f, O = 0.0f;
    for (int s = 0; s < p.n_split; s++) {
        const float *ps = pbase + s * stride;
        const float f = (ps[0] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(ps[0] - M);
        L = fmaf(ps[1], f, L);
        O = fmaf(ps[2 + c], f, O);
    }
    const size_t oi = ((size_t)b * p.n_kv_heads * G + (size_t)kvh * G + h) * D + c;
    p.out[oi] = L > 0.0f ? O / L : 0.0f;
}

template <int D, int G, int KF>
hipError_t launch_one(int units, const DecodeParams &p, hipStream_t s)
{
    dim3 grid((unsigned)p.n_split, (unsigned)units), block(kWave);
    hipLaunchKernelGGL((decode_kernel<D, G, KF>), grid, block, 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1)
        return e;
    dim3 mgrid((unsigned)G, (unsigned)units), mblock(D);
    hipLaunchKernelGGL((merge_kernel<D, G>), mgrid, mblock, 0, s, p);
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

template <int D, int G, int KF>
const void *kernel_of() { return reinterpret_cast<const void *>(&decode_kernel<D, G, KF>); }

template <int D, int G>
const void *kernel_kf(int kfmt)
{
    return kfmt == KVQ_K_ASYM2 ? kernel_of<D, G, KVQ_K_ASYM2>()
           : kfmt == KVQ_K_ASYM4 ? kernel_of<D, G, KVQ_K_ASYM4>()
                                 : kernel_of<D, G, KVQ_K_LLOYD4>();
}

template <int D>
const void *kernel_g(int group, int kfmt)
{
    return group == 1 ? kernel_kf<D, 1>(kfmt) : group == 2 ? kernel_kf<D, 2>(kfmt)
           : group == 4 ? kernel_kf<D, 4>(kfmt) : kernel_kf<D, 8>(kfmt);
}

} // namespace

int decode_slots(int head_dim, int group, int kfmt)
{
    // resident one-wave workgroups of this instantiation on the current device, cached;
    // 256 CUs x 8 when the runtime cannot be asked (no device)
    static std::atomic<int> cache[2][4][3];
    const int di = head_dim == 128 ? 1 : 0;
    const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : 3;
    const int ki = kfmt < 0 ? 0 : kfmt > 2 ? 2 : kfmt;
    int v = cache[di][gi][ki].load();
    if (v > 0)
        return v;
    int dev = 0, cus = 0, per_cu = 0;
    const void *k = head_dim == 128 ? kernel_g<128>(group, kfmt) : kernel_g<64>(group, kfmt);
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kWave, 0) == hipSuccess && cus > 0 &&
        per_cu > 0) {
        v = cus * per_cu;
    } else {
        (void)hipGetLastError();
        v = 256 * 8;
    }
    cache[di][gi][ki].store(v);
    return v;
}

hipError_t launch_decode(int head_dim, int group, int kfmt, int units, const DecodeParams &p,
                         hipStream_t s)
{
    if (head_dim == 128)
        return launch_g<128>(group, kfmt, units, p, s);
    return launch_g<64>(group, kfmt, units, p, s);
}

} // namespace kvq
