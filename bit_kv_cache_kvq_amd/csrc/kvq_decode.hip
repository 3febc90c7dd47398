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
// Three kernels per decode call:
//   qprep   one wave per (sequence, KV head): query in stored coordinates, pruning mask and
//           the integer / fp16 query operands, written once to a small per-unit record.
//   decode  one wave per (unit, context split); the host sizes the splits so every SIMD
//           slot the kernel's register use allows holds a wave.  The query record is read
//           with uniform loads, so its operands sit in scalar registers.
//           * score phase, lane per position: each lane scores 2 consecutive positions; a
//             key row is one dwordx2 load per lane (512 B contiguous per wave).  Asymmetric
//             codes are spread into bytes by shift+mask and multiplied with v_dot4_i32_i8
//             against the query held as a 16-bit integer in two signed-byte planes: exact
//             int32 sums, and the zero-point term uses the same integer query, so code and
//             zero terms together equal q_int . k^ with no cancellation between them
//             (heavy-tailed keys make the group zero large).  Lloyd-Max codes go through an
//             LDS table of fp16 centroid pairs and v_dot2_f32_f16 against fp16 query pairs.
//           * softmax: a running maximum per head; a wave-wide DPP reduction and a rescale
//             happen only when a tile holds a logit above it (rare after the first tiles).
//           * value phase, lane per 8 channels: v_dot2_f32_f16 over position pairs (value
//             words interleave two positions); a 4-bit code masked into the low mantissa
//             bits of a half is the subnormal integer code * 2^-24 (or * 2^-20), so no
//             conversion is needed.  The fp16 weights p*s of a position pair and scale
//             group reach the value lanes through LDS, all heads in one 16-byte read.
//           * the next tile's key-side words are loaded before the value phase of the
//             current one; cache reads are non-temporal (each byte is read once).
//   merge   combines the per-split partial softmax states (skipped for one split).
// No MFMA: this is a bandwidth-bound scan.
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
    static constexpr int CPL = D / 64;             // channels per lane in the query prep
    static constexpr int WV = (G + 3) / 4;         // uint4 of fp16 weight pairs per (group, pair)
    // query record, u32 words per unit: mask; per head the accumulator unit (log2-logit
    // per accumulator step) and the channel-0 coefficient; zero-term sums [G][NG]; query
    // operands [KROWS][G][QW]; scaled masked fp32 query [G][D] (sink positions)
    static constexpr int OFF_MASK = 0;
    static constexpr int OFF_QSC = 4;
    static constexpr int OFF_Q0 = OFF_QSC + G;
    static constexpr int OFF_QZ = OFF_Q0 + G;
    static constexpr int OFF_QP = (OFF_QZ + G * NG + 7) / 8 * 8;
    static constexpr int OFF_QF = OFF_QP + KROWS * G * QW;
    static constexpr int QREC = (OFF_QF + G * D + 63) / 64 * 64;
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

// Cache reads are raw buffer loads: one descriptor per (unit, array) holds the unit's slab
// (base, byte size), the lane part of the offset is a VGPR and the position part an SGPR,
// so no 64-bit address arithmetic runs on the VALU.  An access at or beyond the slab size
// returns zero without touching memory; a descriptor of size 0 turns a prefetch past the
// last tile into a no-op without a branch.  All of them are non-temporal (read once).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
constexpr int kBufWord3 = 0x00020000; // raw 32-bit access, no format conversion
constexpr int kNonTemporal = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ uint2 bload2(rsrc_t r, uint32_t voff, uint32_t soff)
{
    const u2v t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNonTemporal);
    return make_uint2(t.x, t.y);
}
__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNonTemporal);
}

// ===================================================================== query prep
// One wave per unit: stored-coordinate query (FWHT when keys are rotated), 16-channel
// group energies (fp32 stride-halving tree, the order the format fixes), mask, and the
// query operands of the decode kernel.
template <int D, int G, int KF>
__global__ __launch_bounds__(kWave) void qprep_kernel(DecodeParams p)
{
    using C = Cfg<D, G, KF>;
    constexpr int KB = C::KB, KROWS = C::KROWS, PPW = C::PPW, NG = C::NG, NP = C::NP;
    constexpr int CPL = C::CPL, QW = C::QW;
    __shared__ float sq_[G][D];
    __shared__ float se[G][NP];
    __shared__ float sam[G][NP];

    const int lane = threadIdx.x;
    const int unit = blockIdx.x;
    const int b = unit / p.n_kv_heads;
    const int kvh = unit % p.n_kv_heads;
    const int n_q_heads = p.n_kv_heads * G;
    uint32_t *rec = p.qprep + (size_t)unit * C::QREC;
    float *recf = reinterpret_cast<float *>(rec);

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
            sq_[h][lane * CPL + s] = y[s];
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
            se[h][lane / (16 / CPL)] = e;
            sam[h][lane / (16 / CPL)] = am;
        }
    }
    __syncthreads();

    // mask: keep the `keep` highest group energies summed over the heads in ascending
    // head order, ties to the lower group
    uint32_t mask = (1u << NP) - 1u;
    if (p.keep > 0 && p.keep < NP) {
        float E[NP];
#pragma unroll
        for (int g = 0; g < NP; g++) {
            float acc = se[0][g];
#pragma unroll
            for (int h = 1; h < G; h++)
                acc = acc + se[h][g];
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
    if (lane == 0) {
        rec[C::OFF_MASK] = mask;
        if (p.mask_out)
            p.mask_out[unit] = (uint8_t)mask;
    }
    const float qscale = p.sm_log2e / (p.rotate ? (float)D : 1.0f);

    // scaled, masked fp32 query (the sink positions use it directly)
    for (int h = 0; h < G; h++) {
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            const int c = lane * CPL + s;
            const bool kept = (mask >> (c / 16)) & 1u;
            const float v = kept ? sq_[h][c] * qscale : 0.0f;
            sq_[h][c] = v;
            recf[C::OFF_QF + h * D + c] = v;
        }
    }
    __syncthreads();

    if constexpr (KF == KVQ_K_LLOYD4) {
        // fp16 pairs scaled so the largest kept |q| lands in [2^12, 2^13); byte j of key
        // word r holds channels (8r + 2j, 8r + 2j + 1)
        float amax = 0.0f;
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int g = 0; g < NP; g++)
                if (mask >> g & 1u)
                    amax = fmaxf(amax, sam[h][g]);
        amax *= qscale;
        int ex = 0;
        (void)frexpf(amax, &ex);
        const float g2 = amax > 0.0f ? ldexpf(1.0f, 13 - ex) : 1.0f;
        for (int h = 0; h < G; h++) {
            if (lane < KROWS * PPW) {
                const int r = lane / PPW, j = lane % PPW;
                const int ca = 8 * r + 2 * j;
                rec[C::OFF_QP + (r * G + h) * QW + j] = pack_f16x2(sq_[h][ca] * g2, sq_[h][ca + 1] * g2);
            }
            if (lane == 0) {
                recf[C::OFF_QSC + h] = 1.0f / g2;
                recf[C::OFF_Q0 + h] = 0.0f;
            }
        }
    } else {
        for (int h = 0; h < G; h++) {
            // 16-bit integer query: q ~= qi * unit, |qi| <= 32639, written as 256*hi + lo
            // with signed bytes hi, lo.  Channel 0 is scored from its BF16 copy instead.
            float am = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < CPL; s2++) {
                const int c = lane * CPL + s2;
                if (!(p.ch0 && c == 0))
                    am = fmaxf(am, fabsf(sq_[h][c]));
            }
            am = wave_max_dpp(am);
            const float unit_q = am > 0.0f ? am / 32639.0f : 1.0f;
            const float inv = 1.0f / unit_q;
            // key word r, spread register k: byte m holds channel r*(32/KB) + m*(KB==2 ? 4 : 2) + k;
            // words per (row, head): hi planes of registers 0..NREG-1, then the lo planes
            if (lane < KROWS * C::NREG) {
                const int r = lane / C::NREG, k = lane % C::NREG;
                uint32_t hi = 0, lo = 0;
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    const int c = (KB == 2) ? 16 * r + 4 * m + k : 8 * r + 2 * m + k;
                    const float qv = (p.ch0 && c == 0) ? 0.0f : sq_[h][c];
                    const int qi = (int)__builtin_rintf(qv * inv);
                    const int h8 = (qi + 128) >> 8;
                    const int l8 = qi - 256 * h8;
                    hi |= (uint32_t)(h8 & 0xFF) << (8 * m);
                    lo |= (uint32_t)(l8 & 0xFF) << (8 * m);
                }
                rec[C::OFF_QP + (r * G + h) * QW + k] = hi;
                rec[C::OFF_QP + (r * G + h) * QW + C::NREG + k] = lo;
            }
            if (lane < NG) {
                float si = 0.0f;
                for (int c = 32 * lane; c < 32 * lane + 32; c++)
                    if (!(p.ch0 && c == 0))
                        si += __builtin_rintf(sq_[h][c] * inv);
                recf[C::OFF_QZ + h * NG + lane] = si;
            }
            if (lane == 0) {
                recf[C::OFF_QSC + h] = unit_q;
                recf[C::OFF_Q0 + h] = (p.ch0 && (mask & 1u)) ? sq_[h][0] * inv : 0.0f;
            }
        }
    }
}

// ===================================================================== decode
template <int D, int G, int KF>
struct Smem {
    using C = Cfg<D, G, KF>;
    uint32_t lut[KF == KVQ_K_LLOYD4 ? 256 : 1];      // Lloyd-Max code-pair table (fp16x2)
    float sink_p[G][kMaxSink];
    uint4 w[C::NG][C::PAIRS + 1][C::WV];             // fp16 weight pairs: [group][pair][heads]
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

// Descriptors of one unit's slabs.
struct Slabs {
    rsrc_t kc, ksz, kx, vsz, vc;
};

template <int D, int G, int KF>
__device__ __forceinline__ void load_ktile(KTile<D, G, KF> &k, const Slabs &sl, uint32_t cap, int lane, int t0,
                                           uint32_t mask)
{
    using C = Cfg<D, G, KF>;
    const uint32_t vo = (uint32_t)lane * C::TPL * 4u;  // lane's 2 positions of a u32 row
#pragma unroll
    for (int r = 0; r < C::KROWS; r++)
        if (mask >> (r / C::RPP) & 1u)
            k.kc[r] = bload2(sl.kc, vo, ((uint32_t)r * cap + (uint32_t)t0) * 4u);
    if constexpr (KF != KVQ_K_LLOYD4) {
#pragma unroll
        for (int g = 0; g < C::NG; g++)
            if (mask >> (2 * g) & 3u)
                k.ksz[g] = bload2(sl.ksz, vo, ((uint32_t)g * cap + (uint32_t)t0) * 4u);
        k.kx = 0;
        if (mask & 1u)
            k.kx = bload1(sl.kx, vo / 2u, (uint32_t)t0 * 2u);
    } else {
        k.kx = bload1(sl.kx, vo / 2u, (uint32_t)t0 * 2u);
    }
#pragma unroll
    for (int g = 0; g < C::NG; g++)
        k.vsz[g] = bload2(sl.vsz, vo, ((uint32_t)g * cap + (uint32_t)t0) * 4u);
}

// Asymmetric-key logits of this lane's TPL positions in accumulator units:
//   lg = sum_g s_g * (q_int . code)_g + z_g * sum_{c in g} q_int_c  (+ k0 * q0)
// ALL: every 16-channel row is kept (no pruning), so the row tests fold away.
// Per (group, head, position) one int32 sum collects the hi-plane products, is shifted
// by 8, then collects the lo-plane products: sum = 256 * hi.code + lo.code = q_int.code.
// The query operands are uniform loads from the unit's record.
template <int D, int G, int KF, bool ALL>
__device__ __forceinline__ void score_asym(const KTile<D, G, KF> &cur, const uint32_t *__restrict__ rec,
                                           uint32_t mask, int ch0, float (&lg)[Cfg<D, G, KF>::TPL][G])
{
    using C = Cfg<D, G, KF>;
    constexpr int KB = C::KB, KROWS = C::KROWS, NG = C::NG, TPL = C::TPL, NREG = C::NREG, QW = C::QW;
    constexpr int RPG = KROWS / NG; // key rows per scale group
    const float *recf = reinterpret_cast<const float *>(rec);
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
#pragma unroll
                    for (int k = 0; k < NREG; k++) {
                        const int qv = (int)rec[C::OFF_QP + (r * G + h) * QW + plane * NREG + k];
#pragma unroll
                        for (int i = 0; i < TPL; i++)
                            acc[i] = __builtin_amdgcn_sdot4(qv, (int)bsp[rr][i][k], acc[i], false);
                    }
                }
            }
            const float qz = recf[C::OFF_QZ + h * NG + g];
#pragma unroll
            for (int i = 0; i < TPL; i++) {
                const uint32_t szw = i == 0 ? cur.ksz[g].x : cur.ksz[g].y;
                lg[i][h] = fmaf(hi_f16(szw), qz, fmaf(lo_f16(szw), (float)acc[i], lg[i][h]));
            }
        }
    }
    if (ch0 && (mask & 1u)) {
#pragma unroll
        for (int i = 0; i < TPL; i++) {
            const float k0 = bf16_to_f32(i == 0 ? (cur.kx & 0xFFFFu) : (cur.kx >> 16));
#pragma unroll
            for (int h = 0; h < G; h++)
                lg[i][h] = fmaf(k0, recf[C::OFF_Q0 + h], lg[i][h]);
        }
    }
}

// Register budget: 4 heads over INT2 keys fit 3 waves per SIMD (168 VGPRs); 4-bit keys
// (twice the key words in flight) and 8 heads get 2.
template <int D, int G, int KF>
__global__ __launch_bounds__(kWave)
__attribute__((amdgpu_waves_per_eu((G < 4 || (G == 4 && KF == KVQ_K_ASYM2)) ? 3 : 2)))
void decode_kernel(DecodeParams p, const uint32_t *__restrict__ qrec)
{
    using C = Cfg<D, G, KF>;
    constexpr int KROWS = C::KROWS, NG = C::NG, NP = C::NP;
    constexpr int TPL = C::TPL, TILE = C::TILE, WPP = C::WPP, LPP = C::LPP, PPI = C::PPI;
    constexpr int VIT = C::VIT, VW = C::VW, WV = C::WV;
    __shared__ Smem<D, G, KF> sm;

    const int lane = threadIdx.x;
    const int split = blockIdx.x;
    const int unit = blockIdx.y;
    const int b = unit / p.n_kv_heads;
    const int kvh = unit % p.n_kv_heads;
    const size_t cap = (size_t)p.cap;
    const int n_q_heads = p.n_kv_heads * G;
    const uint32_t *__restrict__ rec = qrec + (size_t)unit * C::QREC;
    const float *__restrict__ recf = reinterpret_cast<const float *>(rec);

    const uint32_t mask = rec[C::OFF_MASK];
    const bool all_rows = mask == (1u << NP) - 1u;
    float acc_to_logit[G], logit_to_acc[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        acc_to_logit[h] = recf[C::OFF_QSC + h];
        logit_to_acc[h] = 1.0f / acc_to_logit[h];
    }
    if constexpr (KF == KVQ_K_LLOYD4) {
        // code-pair table: byte (lo nibble a, hi nibble b) -> fp16 (cent[a], cent[b])
        for (int e = lane; e < 256; e += kWave)
            sm.lut[e] = pack_f16x2(p.codebook[e & 15], p.codebook[e >> 4]);
        __syncthreads();
    }

    // ------------------------------------------------------------------ state
    const int vs = lane % LPP;         // value slot: channels 8*vs .. 8*vs+7
    const int vgrp = vs / 4;           // its scale group
    float acc[G][8];
    float zacc[G][NG];
    float lsum[G];
    float mrun[G], mthr[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        lsum[h] = 0.0f;
        mrun[h] = -__builtin_inff();
        mthr[h] = -__builtin_inff();
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
                    sl[h] = fmaf(recf[C::OFF_QF + h * D + c + 1], k1, fmaf(recf[C::OFF_QF + h * D + c], k0, sl[h]));
            }
        }
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float x = valid ? sl[h] : -__builtin_inff();
            mrun[h] = wave_max_dpp(x);
            mthr[h] = mrun[h] * logit_to_acc[h];
            const float pr = valid ? __builtin_amdgcn_exp2f(x - mrun[h]) : 0.0f;
            lsum[h] += pr;
            sm.sink_p[h][lane] = pr;
        }
        __syncthreads();
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
    const uint32_t ucap = (uint32_t)p.cap;
    Slabs sl;
    sl.kc = make_rsrc(p.k_codes + (size_t)unit * KROWS * cap, (uint32_t)KROWS * ucap * 4u);
    sl.vsz = make_rsrc(p.v_sz + (size_t)unit * NG * cap, (uint32_t)NG * ucap * 4u);
    sl.vc = make_rsrc(p.v_codes + (size_t)unit * (cap / 2) * WPP, (ucap / 2u) * WPP * 4u);
    if constexpr (KF != KVQ_K_LLOYD4) {
        sl.ksz = make_rsrc(p.k_sz + (size_t)unit * NG * cap, (uint32_t)NG * ucap * 4u);
        sl.kx = p.ch0 ? make_rsrc(p.k_ch0 + (size_t)unit * cap, ucap * 2u) : make_rsrc(p.k_codes, 0u);
    } else {
        sl.ksz = make_rsrc(p.k_codes, 0u);
        sl.kx = make_rsrc(p.k_norm + (size_t)unit * cap, ucap * 2u);
    }
    const Slabs none = {make_rsrc(p.k_codes, 0u), make_rsrc(p.k_codes, 0u), make_rsrc(p.k_codes, 0u),
                        make_rsrc(p.k_codes, 0u), make_rsrc(p.k_codes, 0u)};
    // value words: lane's pair row and channel slot
    const uint32_t vvo = ((uint32_t)(lane / LPP) * WPP + (uint32_t)(VW * vs)) * 4u;

    // value words of the current tile: word pair `it` is reloaded with the next tile's
    // right after its last use, so each load has a whole tile of work to arrive
    uint2 vcur[VIT];
    KTile<D, G, KF> cur;
    int tile = t_first;
    {
        const Slabs &s0 = tile < t_last ? sl : none;
        load_ktile<D, G, KF>(cur, s0, ucap, lane, tile * TILE, mask);
#pragma unroll
        for (int it = 0; it < VIT; it++)
            vcur[it] = bload2(s0.vc, vvo, ((uint32_t)(tile * TILE / 2 + it * PPI) * WPP) * 4u);
    }
    for (; tile < t_last; tile++) {
        const int t0 = tile * TILE;
        const int tl = t0 + lane * TPL;

        // ---- scores (accumulator units; log2 logit = lg * acc_to_logit[h])
        float lg[TPL][G];
#pragma unroll
        for (int i = 0; i < TPL; i++)
#pragma unroll
            for (int h = 0; h < G; h++)
                lg[i][h] = 0.0f;
        if constexpr (KF != KVQ_K_LLOYD4) {
            if (all_rows)
                score_asym<D, G, KF, true>(cur, rec, mask, p.ch0, lg);
            else
                score_asym<D, G, KF, false>(cur, rec, mask, p.ch0, lg);
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
                for (int h = 0; h < G; h++)
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const uint32_t qv = rec[C::OFF_QP + (r * G + h) * C::QW + j];
#pragma unroll
                        for (int i = 0; i < TPL; i++)
                            lg[i][h] = dot2(pr[i][j], qv, lg[i][h]);
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

        // ---- value scale/zero of this lane's positions; positions outside [q_lo, q_hi)
        // get logit -inf and scale/zero 0 (their slots may hold anything)
        uint32_t vsw[TPL][NG];
#pragma unroll
        for (int g = 0; g < NG; g++) {
            vsw[0][g] = cur.vsz[g].x;
            vsw[1][g] = cur.vsz[g].y;
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
                    for (int g = 0; g < NG; g++)
                        vsw[i][g] = 0u;
                }
            }
        }

        // ---- next tile's key-side words, into the registers this tile no longer needs:
        // in flight during the rest of this tile
        const Slabs &nx = tile + 1 < t_last ? sl : none;
        load_ktile<D, G, KF>(cur, nx, ucap, lane, t0 + TILE, mask);

        // ---- online softmax (log2 units); wave-wide max only when some logit exceeds
        // the running maximum
        // (the test compares in accumulator units against mthr = mrun / acc_to_logit; a
        // rounding miss only lets a weight exceed 1 by an ulp)
        uint64_t above = 0;
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int i = 0; i < TPL; i++)
                above |= __ballot(lg[i][h] > mthr[h]);
        if (above) {
#pragma unroll
            for (int h = 0; h < G; h++) {
                float mt = lg[0][h];
#pragma unroll
                for (int i = 1; i < TPL; i++)
                    mt = fmaxf(mt, lg[i][h]);
                const float mnew = fmaxf(mrun[h], wave_max_dpp(mt * acc_to_logit[h]));
                const float alpha = __builtin_amdgcn_exp2f(mrun[h] - mnew);
                mrun[h] = mnew;
                mthr[h] = mnew * logit_to_acc[h];
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
        // zero-point term and the fp16 weights p*s of this lane's position pair (-> LDS),
        // from the weights rounded to fp16 pairs: one packed product and one dot2 per
        // (group, head)
        uint32_t ph[G];
#pragma unroll
        for (int h = 0; h < G; h++)
            ph[h] = pack_f16x2(pw[0][h], pw[1][h]);
#pragma unroll
        for (int g = 0; g < NG; g++) {
            const uint32_t sp = __builtin_amdgcn_perm(vsw[1][g], vsw[0][g], 0x05040100u); // (s0, s1)
            const uint32_t zp = __builtin_amdgcn_perm(vsw[1][g], vsw[0][g], 0x07060302u); // (z0, z1)
            uint32_t wq[4 * WV];
#pragma unroll
            for (int h = 0; h < G; h++) {
                zacc[h][g] = dot2(ph[h], zp, zacc[h][g]);
                wq[h] = mul_f16x2(ph[h], sp);
            }
#pragma unroll
            for (int h = G; h < 4 * WV; h++)
                wq[h] = 0u;
#pragma unroll
            for (int v4 = 0; v4 < WV; v4++)
                sm.w[g][lane][v4] = make_uint4(wq[4 * v4], wq[4 * v4 + 1], wq[4 * v4 + 2], wq[4 * v4 + 3]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- values: lane owns channels 8*vs .. 8*vs+7 of one pair per iteration
        const uint32_t vnext = (uint32_t)((t0 + TILE) / 2) * WPP * 4u;
#pragma unroll
        for (int it = 0; it < VIT; it++) {
            const uint2 vv = vcur[it];
            vcur[it] = bload2(nx.vc, vvo, vnext + (uint32_t)(it * PPI * WPP) * 4u);
            const int pl = it * PPI + lane / LPP;
            uint32_t wv[4 * WV];
#pragma unroll
            for (int v4 = 0; v4 < WV; v4++) {
                const uint4 t4 = sm.w[vgrp][pl][v4];
                wv[4 * v4 + 0] = t4.x;
                wv[4 * v4 + 1] = t4.y;
                wv[4 * v4 + 2] = t4.z;
                wv[4 * v4 + 3] = t4.w;
            }
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

// ===================================================================== split merge
// One thread per (sequence, query head, channel) combines the per-split (m, l, o) partials:
// one global softmax over all positions (Dual-QK sec. 3.4).
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

// ===================================================================== launchers
template <int D, int G, int KF>
hipError_t launch_one(int units, const DecodeParams &p, hipStream_t s)
{
    hipLaunchKernelGGL((qprep_kernel<D, G, KF>), dim3((unsigned)units), dim3(kWave), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((decode_kernel<D, G, KF>), dim3((unsigned)p.n_split, (unsigned)units), dim3(kWave), 0, s,
                       p, static_cast<const uint32_t *>(p.qprep));
    e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1)
        return e;
    hipLaunchKernelGGL((merge_kernel<D, G>), dim3((unsigned)G, (unsigned)units), dim3(D), 0, s, p);
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

template <int D, int G>
int qrec_kf(int kfmt)
{
    return kfmt == KVQ_K_ASYM2 ? Cfg<D, G, KVQ_K_ASYM2>::QREC
           : kfmt == KVQ_K_ASYM4 ? Cfg<D, G, KVQ_K_ASYM4>::QREC
                                 : Cfg<D, G, KVQ_K_LLOYD4>::QREC;
}

template <int D>
int qrec_g(int group, int kfmt)
{
    return group == 1 ? qrec_kf<D, 1>(kfmt) : group == 2 ? qrec_kf<D, 2>(kfmt)
           : group == 4 ? qrec_kf<D, 4>(kfmt) : qrec_kf<D, 8>(kfmt);
}

} // namespace

int decode_qrec_words(int head_dim, int group, int kfmt)
{
    return head_dim == 128 ? qrec_g<128>(group, kfmt) : qrec_g<64>(group, kfmt);
}

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
