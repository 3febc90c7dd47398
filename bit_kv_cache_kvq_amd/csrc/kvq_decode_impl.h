// kvq_decode_impl.h -- decode attention scored straight from the packed low-bit cache.
// (Kernel templates; kvq_decode.hip and kvq_decode_v2.hip instantiate them for the two value
// formats, in parallel compilations.)
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
//   * one softmax over all positions (Dual-QK sec. 3.4), computed online by each wave over
//     its tiles; the waves sharing a unit combine their states at the end (the last one to
//     finish does it, after an agent-scope release / acquire on a per-unit counter);
//   * values from INT4 codes per 32-channel group, or per-token INT2 codes (Dual-QK sec.
//     B.2): o = sum_t p_t s_{t,g} code_{t,c} + sum_t p_t z_{t,g}.
//
// Two kernels per decode call:
//   qprep   one workgroup per (sequence, KV head), one wave per query head: query in stored
//           coordinates, pruning mask, the integer / fp16 query operands and the sink
//           positions' softmax state, written once to a small per-unit record.
//   decode  one wave per resident SIMD slot (at least one per unit); the waves serving a
//           unit draw its 128-position tiles from a counter.  The query record is read
//           with uniform loads, so its operands sit in scalar registers.
//           * score phase, lane per position: each lane scores 2 consecutive positions; a
//             key row is one dwordx2 load per lane (512 B contiguous per wave).  Asymmetric
//             codes are spread into bytes by shift+mask and multiplied with v_dot4_i32_i8
//             against the query held as a 16-bit integer (14 bits of magnitude for INT2
//             keys, whose spread bytes carry code or 4*code) in two signed-byte planes: exact
//             int32 sums, and the zero-point term uses the same integer query, so code and
//             zero terms together equal q_int . k^ with no cancellation between them
//             (heavy-tailed keys make the group zero large).  Lloyd-Max codes go through an
//             LDS table of fp16 centroid pairs and v_dot2_f32_f16 against fp16 query pairs.
//           * softmax: a running maximum per head; a wave-wide DPP reduction and a rescale
//             happen only when a tile holds a logit well above it (rare after the first
//             tiles).
//           * value phase, lane per 8 channels: v_dot2_f32_f16 over position pairs (value
//             words interleave two positions); a 4-bit code masked into the low mantissa
//             bits of a half is the subnormal integer code * 2^-24 (or * 2^-20), so no
//             conversion is needed.  The fp16 weights p*s of a position pair and scale
//             group reach the value lanes through LDS, all heads in one 16-byte read.
//           * the next tile's key-side words are loaded before the value phase of the
//             current one; cache reads are non-temporal (each byte is read once).
// No MFMA: this is a bandwidth-bound scan.
#pragma once

#include <atomic>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int D, int G, int KF, int VF = KVQ_V_ASYM4_G32>
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
    static constexpr int NGV = VF == KVQ_V_ASYM4_G32 ? D / 32 : 1;  // value scale groups
    static constexpr int NWG = VF == KVQ_V_KQV ? 2 : NGV;              // weight sets (KQV: rho, residual norm)
    static constexpr int WPP = VF == KVQ_V_ASYM2_TOKEN ? D / 8 : D / 4; // value words per position pair
    static constexpr int VW = VF == KVQ_V_ASYM2_TOKEN ? 1 : 2;          // value words per lane per iteration
    static_assert(WPP / VW * 8 == D, "a value lane owns 8 channels");
    static constexpr int LPP = WPP / VW;           // value lanes per pair
    static constexpr int PPI = 64 / LPP;           // pairs per value iteration
    static constexpr int VIT = PAIRS / PPI;        // value iterations per tile
    static constexpr int CPL = D / 64;             // channels per lane in the query prep
    static constexpr int WV = (G + 3) / 4;         // uint4 of fp16 weight pairs per (group, pair)
    // query record, u32 words per unit: mask; per head the accumulator unit (log2-logit
    // per accumulator step) and the channel-0 coefficient; zero-term sums [G][NG]; query
    // operands [KROWS][G][QW]; the softmax state (m, l, o[D]) of the BF16 sink positions
    // per head [G][D + 2]
    static constexpr int OFF_MASK = 0;
    static constexpr int OFF_QSC = 4;
    static constexpr int OFF_Q0 = OFF_QSC + G;
    static constexpr int OFF_QZ = OFF_Q0 + G;
    static constexpr int OFF_QP = (OFF_QZ + G * NG + 7) / 8 * 8;
    static constexpr int OFF_SINK = OFF_QP + KROWS * G * QW;
    static constexpr int QREC = (OFF_SINK + G * (D + 2) + 63) / 64 * 64;
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

template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_add_step(float x)
{
    const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWMASK, 0xF, false);
    return x + __int_as_float(o);
}

// sum over the wave, result uniform (DPP row shifts, then row broadcasts to lane 63)
__device__ __forceinline__ float wave_sum_dpp(float v)
{
    v = dpp_add_step<0x111, 0xF>(v); // row_shr:1
    v = dpp_add_step<0x112, 0xF>(v); // row_shr:2
    v = dpp_add_step<0x114, 0xF>(v); // row_shr:4
    v = dpp_add_step<0x118, 0xF>(v); // row_shr:8
    v = dpp_add_step<0x142, 0xA>(v); // row_bcast:15
    v = dpp_add_step<0x143, 0xC>(v); // row_bcast:31
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

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// Cache reads are raw buffer loads: one descriptor per (unit, array) holds the unit's slab
// (base, byte size below 2^30), the lane part of the offset is a VGPR and the position part
// an SGPR, so no 64-bit address arithmetic runs on the VALU.  An access whose lane offset
// is at or beyond the slab size returns zero without touching memory: adding kNoAccess to
// the lane offset turns a prefetch past the last tile into a no-op without a branch.  All
// of them are non-temporal (read once).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
constexpr int kBufWord3 = 0x00020000; // raw 32-bit access, no format conversion
constexpr int kNonTemporal = 2;
constexpr uint32_t kNoAccess = 0x80000000u;
// log2 slack of the lazily raised softmax maximum (weights stay below 2^kSlack)
constexpr float kSlack = 2.0f;

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
// a lane's value words of one position pair: two (INT4) or one (per-token INT2)
template <bool ONE>
__device__ __forceinline__ std::conditional_t<ONE, uint32_t, uint2> vload(rsrc_t r, uint32_t voff, uint32_t soff)
{
    if constexpr (ONE)
        return bload1(r, voff, soff);
    else
        return bload2(r, voff, soff);
}

// ===================================================================== query prep
// One workgroup per unit, one wave per query head of the GQA group: stored-coordinate query
// (FWHT when keys are rotated), 16-channel group energies (fp32 stride-halving tree, the
// order the format fixes), the group's mask, and the head's query operands and sink state.
template <int D, int G, int KF, int SB>
__global__ __launch_bounds__(kWave * G) void qprep_kernel(DecodeParams p)
{
    using C = Cfg<D, G, KF>;
    constexpr int KB = C::KB, KROWS = C::KROWS, PPW = C::PPW, NG = C::NG, NP = C::NP;
    constexpr int CPL = C::CPL, QW = C::QW;
    __shared__ float sq_[G][D];
    __shared__ float se[G][NP];
    __shared__ float sam[G][NP];
    __shared__ float sp[G][kWave];

    const int lane = threadIdx.x % kWave;
    const int h = (int)uniform(threadIdx.x / kWave); // this wave's head
    // workgroups of bucket 0 first: they also compute the BF16 positions' softmax state, the
    // longest work of the kernel, so they start before the other buckets' records
    const int bk = (int)blockIdx.x / p.n_units; // bucket of this record (0 without RoPE)
    const int unit = (int)blockIdx.x % p.n_units;
    const int b = unit / p.n_kv_heads;
    const int kvh = unit % p.n_kv_heads;
    const int n_q_heads = p.n_kv_heads * G;
    const bool state = bk == 0; // this workgroup also computes the BF16 positions' state
    uint32_t *rec = p.qprep + ((size_t)unit * p.n_rb + bk) * C::QREC;
    float *recf = reinterpret_cast<float *>(rec);

    // BF16 sink rows, SB at a time (the last row repeated past n_sink); the first batch of
    // keys and values is loaded here, with the query, so its latency overlaps the query's.
    // SB is 8, or 32 for more than 8 sinks (64 sinks then cost two rounds of latency).
    const int n_sink = p.n_sink < p.len ? p.n_sink : p.len;
    auto load_sinks = [&](const uint16_t *base, int t0, float (&dst)[SB][CPL]) {
#pragma unroll
        for (int j = 0; j < SB; j++) {
            const int t = t0 + j < n_sink ? t0 + j : n_sink - 1;
            const uint16_t *row = base + ((size_t)unit * p.n_sink + t) * D + lane * CPL;
#pragma unroll
            for (int s = 0; s < CPL; s++)
                dst[j][s] = bf16_to_f32(row[s]);
        }
    };
    float kv[SB][CPL], vv[SB][CPL];
    if (state && n_sink > 0) {
        load_sinks(p.sink_k, 0, kv);
        load_sinks(p.sink_v, 0, vv);
    }

    float yq[CPL]; // this head's query as given
    {
        const size_t qoff = ((size_t)b * n_q_heads + (size_t)kvh * G + h) * D + (size_t)lane * CPL;
        if (p.q_bf16) {
            const uint16_t *qb = static_cast<const uint16_t *>(p.q) + qoff;
#pragma unroll
            for (int s = 0; s < CPL; s++)
                yq[s] = bf16_to_f32(qb[s]);
        } else {
            const float *qf = static_cast<const float *>(p.q) + qoff;
#pragma unroll
            for (int s = 0; s < CPL; s++)
                yq[s] = qf[s];
        }
    }
    const float qscale = p.sm_log2e / (p.rotate ? (float)D : 1.0f);

    // The query of bucket bq in stored coordinates (rotated back by the bucket's anchor under
    // bucket-relative RoPE, Dual-QK sec. 3.4 / C.4; then Walsh-Hadamard when keys are rotated),
    // its group energies, the mask, and this head's scaled, masked query in qr and sq_[h].
    // Every wave of the workgroup calls it together (two barriers).
    float qr[CPL];
    auto prep = [&](int bq) -> uint32_t {
        float y[CPL];
#pragma unroll
        for (int s = 0; s < CPL; s++)
            y[s] = yq[s];
        if (p.rope_lw)
            anchor_rotate<CPL>(y, p.rope_cs + (size_t)bq * D, lane);
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
        __syncthreads();

        // mask (every wave computes the same one): keep the `keep` highest group energies
        // summed over the heads in ascending head order, ties to the lower group
        uint32_t mask = (1u << NP) - 1u;
        if (p.keep > 0 && p.keep < NP) {
            float E[NP];
#pragma unroll
            for (int g = 0; g < NP; g++) {
                float acc = se[0][g];
#pragma unroll
                for (int hh = 1; hh < G; hh++)
                    acc = acc + se[hh][g];
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

        // this head's scaled, masked fp32 query
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            const int c = lane * CPL + s;
            const bool kept = (mask >> (c / 16)) & 1u;
            qr[s] = kept ? sq_[h][c] * qscale : 0.0f;
            sq_[h][c] = qr[s];
        }
        __syncthreads();
        return mask;
    };
    const uint32_t mask = prep(bk);

    if (state) {
        // the decode kernel's tile and arrival counters of this unit's stripes, at the places
        // u + k * units
        for (int k = threadIdx.x; k < p.n_waves / p.n_units + 1; k += kWave * G)
            if (unit + k * p.n_units < p.n_waves) {
                p.tile_ctr[unit + k * p.n_units] = 0u;
                p.tile_ctr[p.n_waves + unit + k * p.n_units] = 0u;
            }
        if (threadIdx.x == 0)
            p.tile_ctr[2 * p.n_waves + unit] = 0u; // the decode kernel's count of this unit's members done
    }
    if (threadIdx.x == 0) {
        rec[C::OFF_MASK] = mask;
        if (p.mask_out)
            p.mask_out[(size_t)unit * p.n_rb + bk] = (uint8_t)mask;
    }

    // ---- the query operands of this record
    if constexpr (KF == KVQ_K_LLOYD4) {
        // fp16 pairs scaled so the largest kept |q| of the group lands in [2^12, 2^13);
        // byte j of key word r holds channels (8r + 2j, 8r + 2j + 1)
        float amax = 0.0f;
#pragma unroll
        for (int hh = 0; hh < G; hh++)
#pragma unroll
            for (int g = 0; g < NP; g++)
                if (mask >> g & 1u)
                    amax = fmaxf(amax, sam[hh][g]);
        amax *= qscale;
        int ex = 0;
        (void)frexpf(amax, &ex);
        const float g2 = amax > 0.0f ? ldexpf(1.0f, 13 - ex) : 1.0f;
        if (lane < KROWS * PPW) {
            const int r = lane / PPW, j = lane % PPW;
            const int ca = 8 * r + 2 * j;
            rec[C::OFF_QP + (r * G + h) * QW + j] = pack_f16x2(sq_[h][ca] * g2, sq_[h][ca + 1] * g2);
        }
        if (lane == 0) {
            recf[C::OFF_QSC + h] = 1.0f / g2;
            recf[C::OFF_Q0 + h] = 0.0f;
        }
    } else {
        // Integer query: q ~= qi * unit, written as 256*hi + lo with signed bytes hi, lo.
        // INT2 keys: the decode kernel spreads a code word into bytes holding code or
        // 4*code (masks without shifts for half of them), so the plane entries of the
        // unscaled codes carry 4*qi; every sum is then 4*(q_int . code), |qi| <= 8159.
        // 4-bit keys: plain codes, |qi| <= 32639.  Channel 0 is scored from its BF16 copy.
        float am = 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < CPL; s2++) {
            const int c = lane * CPL + s2;
            if (!(p.ch0 && c == 0))
                am = fmaxf(am, fabsf(qr[s2]));
        }
        am = wave_max_dpp(am);
        constexpr int F = KB == 2 ? 4 : 1;
        const float unit_q = am > 0.0f ? am / (KB == 2 ? 8159.0f : 32639.0f) : 1.0f;
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
                const int qi = (int)__builtin_rintf(qv * inv) * ((KB == 2 && k % 2 == 0) ? 4 : 1);
                const int h8 = (qi + 128) >> 8;
                const int l8 = qi - 256 * h8;
                hi |= (uint32_t)(h8 & 0xFF) << (8 * m);
                lo |= (uint32_t)(l8 & 0xFF) << (8 * m);
            }
            rec[C::OFF_QP + (r * G + h) * QW + k] = hi;
            rec[C::OFF_QP + (r * G + h) * QW + C::NREG + k] = lo;
        }
        // zero-term sums: integer query summed over each 32-channel group (lanes of a
        // group: 32/CPL consecutive lanes; integer-valued floats below 2^24, exact)
        {
            float si = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < CPL; s2++) {
                const int c = lane * CPL + s2;
                if (!(p.ch0 && c == 0))
                    si += __builtin_rintf(qr[s2] * inv);
            }
#pragma unroll
            for (int m = 16 / CPL; m >= 1; m >>= 1)
                si += __shfl_xor(si, m);
            if (lane % (32 / CPL) == 0)
                recf[C::OFF_QZ + h * NG + lane / (32 / CPL)] = si * F;
        }
        if (lane == 0) {
            recf[C::OFF_QSC + h] = unit_q / F;
            recf[C::OFF_Q0 + h] = (p.ch0 && (mask & 1u)) ? sq_[h][0] * inv * F : 0.0f;
        }
    }
    if (!state)
        return;

    // BF16 sink positions (t < min(n_sink, len), all in bucket 0): dense dot over the kept
    // channels, then the head's softmax state over them -- log2 max m, sum l and
    // o = sum_t 2^(l_t - m) v_t -- which the decode kernel folds into the unit's result.
    // Lanes own channels; one wave-wide sum per sink gives its logit, lane t keeps that of
    // sink t.
    {
        float mine = -__builtin_inff();
        for (int t0 = 0; t0 < n_sink; t0 += SB) {
            if (t0 > 0)
                load_sinks(p.sink_k, t0, kv);
#pragma unroll
            for (int j = 0; j < SB; j++) {
                if (t0 + j >= n_sink)
                    break;
                float part = 0.0f;
#pragma unroll
                for (int s = 0; s < CPL; s++)
                    part = fmaf(qr[s], kv[j][s], part);
                const float tot = wave_sum_dpp(part);
                mine = lane == t0 + j ? tot : mine;
            }
        }
        const float m = wave_max_dpp(mine);
        const float pr = lane < n_sink ? __builtin_amdgcn_exp2f(mine - m) : 0.0f;
        sp[h][lane] = pr;
        const float l = wave_sum_dpp(pr);
        __syncthreads();
        float o[CPL];
#pragma unroll
        for (int s = 0; s < CPL; s++)
            o[s] = 0.0f;
        for (int t0 = 0; t0 < n_sink; t0 += SB) {
            if (t0 > 0)
                load_sinks(p.sink_v, t0, vv);
#pragma unroll
            for (int j = 0; j < SB; j++) {
                if (t0 + j >= n_sink)
                    break;
#pragma unroll
                for (int s = 0; s < CPL; s++)
                    o[s] = fmaf(sp[h][t0 + j], vv[j][s], o[s]);
            }
        }
        // recent BF16 window, positions [wlo, len) in ring slots t mod W (Dual-QK sec. 3.3 /
        // 4.1), one bucket's positions at a time (the query of that bucket), 64 positions per
        // chunk, lane j scoring position c0 + j over all channels from its ring row, folded
        // into the state (m, l, o) online
        float M = m, L = l;
        const int wlo = p.q_end > n_sink ? p.q_end : n_sink;
        int qb = 0; // bucket whose query qr / sq_ hold
        for (int s0 = wlo; s0 < p.len;) {
            const int bs = p.rope_lw ? s0 >> p.rope_lw : 0;
            const int s1 = p.rope_lw ? min(p.len, (bs + 1) << p.rope_lw) : p.len;
            if (bs != qb) {
                (void)prep(bs);
                qb = bs;
            }
            for (int c0 = s0; c0 < s1; c0 += kWave) {
                const int nc = s1 - c0 < kWave ? s1 - c0 : kWave; // positions in this chunk
                const bool valid = lane < nc;
                // ring slot of the chunk's position j: slot0 + j, wrapped once at most (the window
                // holds at most W positions); positions past the chunk repeat its last one
                const int slot0 = c0 % p.n_recent;
                auto slot = [&](int j) {
                    const int sl = slot0 + (j < nc ? j : nc - 1);
                    return sl >= p.n_recent ? sl - p.n_recent : sl;
                };
                const uint16_t *krow = p.recent_k + ((size_t)unit * p.n_recent + (size_t)slot(lane)) * D;
                float dot = 0.0f;
#pragma unroll
                for (int c = 0; c < D; c += 8) {
                    const uint4 kw = *reinterpret_cast<const uint4 *>(krow + c);
                    const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        dot = fmaf(sq_[h][c + 2 * e], bf16_to_f32(kk[e] & 0xFFFFu), dot);
                        dot = fmaf(sq_[h][c + 2 * e + 1], bf16_to_f32(kk[e] >> 16), dot);
                    }
                }
                const float lw = valid ? dot : -__builtin_inff();
                const float Mn = fmaxf(M, wave_max_dpp(lw)); // finite: the chunk has a position
                const float fo = M == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
                const float pw = valid ? __builtin_amdgcn_exp2f(lw - Mn) : 0.0f;
                L = fmaf(L, fo, wave_sum_dpp(pw));
#pragma unroll
                for (int s = 0; s < CPL; s++)
                    o[s] *= fo;
                // values, 32 positions per batch of loads (rows past the chunk repeat its last
                // position with weight 0); lane owns channels lane*CPL ..
#pragma unroll
                for (int b0 = 0; b0 < kWave; b0 += 32) {
                    float vw[32][CPL];
#pragma unroll
                    for (int jj = 0; jj < 32; jj++) {
                        const uint16_t *vrow =
                            p.recent_v + ((size_t)unit * p.n_recent + (size_t)slot(b0 + jj)) * D + lane * CPL;
#pragma unroll
                        for (int s = 0; s < CPL; s++)
                            vw[jj][s] = bf16_to_f32(vrow[s]);
                    }
#pragma unroll
                    for (int jj = 0; jj < 32; jj++) {
                        const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), b0 + jj));
#pragma unroll
                        for (int s = 0; s < CPL; s++)
                            o[s] = fmaf(pj, vw[jj][s], o[s]);
                    }
                }
                M = Mn;
            }
            s0 = s1;
        }
        if (lane == 0) {
            recf[C::OFF_SINK + h * (D + 2)] = M;
            recf[C::OFF_SINK + h * (D + 2) + 1] = L;
        }
#pragma unroll
        for (int s = 0; s < CPL; s++)
            recf[C::OFF_SINK + h * (D + 2) + 2 + lane * CPL + s] = o[s];
    }
}

// ===================================================================== decode
template <int D, int G, int KF, int VF>
struct Smem {
    using C = Cfg<D, G, KF, VF>;
    uint32_t lut[KF == KVQ_K_LLOYD4 ? 256 : 1];      // Lloyd-Max code-pair table (fp16x2)
    uint32_t vlut[VF == KVQ_V_KQV ? 256 : 1];        // KQV values: byte (2 nibbles) -> (cent[lo & 7], cent[hi & 7])
    float sink_p[G][kMaxSink];
    union {
        uint4 w[C::NWG][C::PAIRS + 1][C::WV];        // fp16 weight pairs: [group][pair][heads]
        float4 red[2 * kWave];                       // end of the tiles: 64 lanes x 8 floats
    };
};

// Key-side words of one tile for this lane (TPL = 2 positions).
template <int D, int G, int KF, int VF>
struct KTile {
    using C = Cfg<D, G, KF, VF>;
    uint2 kc[C::KROWS];
    uint2 ksz[C::NG];
    uint2 vsz[C::NGV];
    uint32_t kx; // channel-0 bf16 pair (asym + protection) or rho fp16 pair (Lloyd-Max)
};

// Descriptors of one unit's slabs.
struct Slabs {
    rsrc_t kc, ksz, kx, vsz, vc;
};

// off: 0, or kNoAccess to turn every load into a zero without a memory access.  ALL: every
// row is kept; otherwise the rows of pruned groups get kNoAccess too (zeros, no traffic, and
// no branch).  CH0: channel 0 is stored apart in BF16.
template <int D, int G, int KF, int VF, bool ALL, bool CH0>
__device__ __forceinline__ void load_ktile(KTile<D, G, KF, VF> &k, const Slabs &sl, uint32_t cap, int lane, int t0,
                                           uint32_t mask, uint32_t off)
{
    using C = Cfg<D, G, KF, VF>;
    const uint32_t vo = (uint32_t)lane * C::TPL * 4u + off;  // lane's 2 positions of a u32 row
    auto gate = [&](uint32_t bits) { return (ALL || (mask & bits)) ? vo : (vo | kNoAccess); };
#pragma unroll
    for (int r = 0; r < C::KROWS; r++)
        k.kc[r] = bload2(sl.kc, gate(1u << (r / C::RPP)), ((uint32_t)r * cap + (uint32_t)t0) * 4u);
    if constexpr (KF != KVQ_K_LLOYD4) {
#pragma unroll
        for (int g = 0; g < C::NG; g++)
            k.ksz[g] = bload2(sl.ksz, gate(3u << (2 * g)), ((uint32_t)g * cap + (uint32_t)t0) * 4u);
        k.kx = 0;
        if constexpr (CH0)
            k.kx = bload1(sl.kx, ((ALL || (mask & 1u)) ? (vo >> 1) : ((vo >> 1) | kNoAccess)), (uint32_t)t0 * 2u); // u16 row
    } else {
        k.kx = bload1(sl.kx, vo >> 1, (uint32_t)t0 * 2u);
    }
#pragma unroll
    for (int g = 0; g < C::NGV; g++)
        k.vsz[g] = bload2(sl.vsz, vo, ((uint32_t)g * cap + (uint32_t)t0) * 4u);
}

// Asymmetric-key logits of this lane's TPL positions in accumulator units:
//   lg = sum_g s_g * (q_int . code)_g + z_g * sum_{c in g} q_int_c  (+ k0 * q0)
// ALL: every 16-channel row is kept (no pruning), so the row tests fold away.
// Per (group, head, position) one int32 sum collects the hi-plane products, is shifted
// by 8, then collects the lo-plane products: sum = 256 * hi.code + lo.code = q_int.code.
// The query operands are uniform loads from the unit's record.
template <int D, int G, int KF, int VF, bool ALL, bool CH0>
__device__ __forceinline__ void score_asym(const KTile<D, G, KF, VF> &cur, const uint32_t *__restrict__ rec,
                                           uint32_t mask, float (&lg)[Cfg<D, G, KF>::TPL][G])
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
                    // bytes hold code (registers 0, 2) or 4*code (1, 3); the query planes
                    // of registers 0 and 2 carry the matching factor 4
                    const uint32_t y = x >> 4;
                    bsp[rr][i][0] = x & 0x03030303u;
                    bsp[rr][i][1] = x & 0x0C0C0C0Cu;
                    bsp[rr][i][2] = y & 0x03030303u;
                    bsp[rr][i][3] = y & 0x0C0C0C0Cu;
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
    if (CH0 && (ALL || (mask & 1u))) {
#pragma unroll
        for (int i = 0; i < TPL; i++) {
            const float k0 = bf16_to_f32(i == 0 ? (cur.kx & 0xFFFFu) : (cur.kx >> 16));
#pragma unroll
            for (int h = 0; h < G; h++)
                lg[i][h] = fmaf(k0, recf[C::OFF_Q0 + h], lg[i][h]);
        }
    }
}

// Descriptors of unit u's slabs.
template <int D, int G, int KF, int VF>
__device__ __forceinline__ Slabs unit_slabs(const DecodeParams &p, int u)
{
    using C = Cfg<D, G, KF, VF>;
    const size_t cap = (size_t)p.cap;
    const uint32_t ucap = (uint32_t)p.cap;
    Slabs sl;
    sl.kc = make_rsrc(p.k_codes + (size_t)u * C::KROWS * cap, (uint32_t)C::KROWS * ucap * 4u);
    sl.vsz = make_rsrc(p.v_sz + (size_t)u * C::NGV * cap, (uint32_t)C::NGV * ucap * 4u);
    sl.vc = make_rsrc(p.v_codes + (size_t)u * (cap / 2) * C::WPP, (ucap / 2u) * C::WPP * 4u);
    if constexpr (KF != KVQ_K_LLOYD4) {
        sl.ksz = make_rsrc(p.k_sz + (size_t)u * C::NG * cap, (uint32_t)C::NG * ucap * 4u);
        sl.kx = p.ch0 ? make_rsrc(p.k_ch0 + (size_t)u * cap, ucap * 2u) : make_rsrc(p.k_codes, 0u);
    } else {
        sl.ksz = make_rsrc(p.k_codes, 0u);
        sl.kx = make_rsrc(p.k_norm + (size_t)u * cap, ucap * 2u);
    }
    return sl;
}

// Work split (one wave per workgroup, W waves, U units, W >= U).  Wave w takes the place
// x = team_slot(w): it serves unit x mod U as member x / U of that unit's team; the team has
// W / U members, one more for the first W mod U units.  Member k scores tile k first; every
// further tile comes from the unit's counter (tiles team_size, team_size + 1, ... in the
// order the members ask), so a member that gets more issue slots takes more tiles and the
// whole team ends together.  Teams of more than kStripe members work the same way on
// stripes of the unit (see the decode kernel).  In the deterministic mode member k takes
// tiles k, k + n, ... of a team (stripe) of n instead.
__device__ __forceinline__ int team_size(int u, int U, int W) { return W / U + (u < W % U ? 1 : 0); }

// Most waves drawing from one counter: draws on one address are serialized where the atomic
// executes, so a large team (few units, long contexts) is cut into stripes of this many.
constexpr int kStripe = 8;

// Issue priority from a team's progress: the tile a wave is on (tiles are taken in
// increasing order, so it tracks how far the whole team or stripe is), in the bands [0, 1/2),
// [1/2, 3/4), [3/4, 7/8), [7/8, 1) of the unit.  The waves sharing a SIMD otherwise issue
// oldest first, which lets whole teams fall behind others; a team in an earlier band now
// goes first, so teams advance together, and the narrow last band bounds how far apart
// they end.
__device__ __forceinline__ void set_priority_for(int t, int Tu)
{
    const int q = (int)(((long long)t * 8) / Tu); // 0..7, uniform
    if (q < 4)
        __builtin_amdgcn_s_setprio(3);
    else if (q < 6)
        __builtin_amdgcn_s_setprio(2);
    else if (q < 7)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// Place of wave w.  Workgroups are dealt to compute units in turn, so waves w, w + n_cu,
// w + 2 n_cu, ... share a CU, and the older of them get more of its issue slots.  When W is
// a multiple of n_cu the places of one CU's waves are made consecutive (x = (w mod n_cu) *
// (W / n_cu) + w / n_cu): the members of a team, U places apart, then sit on different CUs
// at different ages, and no team gets a much larger or smaller share of the device.
// A wave-uniform integer pinned to a scalar register.  The divisions of the work split run
// on the vector unit; the compiler drops a readfirstlane builtin on values it already knows to
// be uniform, and may then keep the unit's slab descriptors and tile offsets in vector
// registers, which puts a loop around every buffer load (one pass per distinct value).  The
// opaque readfirstlane keeps everything derived from these values scalar.  The compiler does
// not look inside the asm for hazards, so the wait states are part of it: the read of a VGPR
// just written by another vector instruction needs one, and an SGPR written by a vector
// instruction needs up to five before a memory instruction or a lane select may read it.
__device__ __forceinline__ int sgpr(int v)
{
    int r;
    asm volatile("s_nop 4\n\tv_readfirstlane_b32 %0, %1\n\ts_nop 4" : "=s"(r) : "v"(v));
    return r;
}

__device__ __forceinline__ int team_slot(int w, int W, int n_cu)
{
    return (n_cu > 0 && W % n_cu == 0) ? (w % n_cu) * (W / n_cu) + w / n_cu : w;
}

// Next tile number from a unit's counter, called by lane 0 only; the return is read a tile
// later (the library builds this file with the compiler's atomic optimizer off, which would
// otherwise broadcast the result, and wait for it, on the spot).
__device__ __forceinline__ uint32_t draw_tile(uint32_t *ctr)
{
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Partial softmax states pass between the waves of a team (on any compute unit) within the
// kernel.  They are written and read back with the device-coherence cache policy (sc1, as
// the compiler gives agent-scope atomic accesses), so both go to the device-coherent level
// rather than a compute unit's or XCD's own caches, and the writer counts itself in on the
// unit's counter only after its stores have completed.  No cache-wide write-back or
// invalidation is needed.  Stores are 16 bytes per lane, whole lines per wave.
constexpr int kCoherent = 16; // sc1
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_shared2(rsrc_t r, uint32_t byte_off, float a, float b)
{
    const u2v v = {__float_as_uint(a), __float_as_uint(b)};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, kCoherent);
}
__device__ __forceinline__ void store_shared4(rsrc_t r, uint32_t byte_off, float a, float b, float c, float d)
{
    const u4v v = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kCoherent);
}
__device__ __forceinline__ float load_shared(rsrc_t r, uint32_t byte_off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCoherent));
}
// Partial state record of one (wave, head): m, l, two unused words, o[D] (16-byte aligned).
template <int D>
constexpr int part_rec() { return D + 4; }

// Combine the partial softmax states (m, l, o) of a unit's team, member k in slot u + k * U,
// with the sink positions' state: one global softmax over all positions (Dual-QK sec. 3.4),
// normalised into out_u[h][D].  Run by one wave; lane j holds channels j, j + 64 of every
// head.  Members go in batches of NB, all heads at once (48 o loads per lane per batch),
// and the next batch's loads are issued before the current batch is folded in, so a team
// of n members costs about one memory latency plus n / NB load rounds (the tile loop's
// registers are free by then: two batches take 96 VGPRs).  Lane j < G * NB reads (m, l)
// of head j / NB, member j % NB of the batch; readlane passes them on.
template <int D, int G>
struct CombineBatch {
    static constexpr int CPL = D / 64;
    static constexpr int NB = 48 / (G * CPL);
    float m, l;
    float o[G][NB][CPL];
};

template <int D, int G>
__device__ __forceinline__ void load_batch(CombineBatch<D, G> &b, rsrc_t r, uint32_t ub, uint32_t stride, int k0,
                                           int team, int lane)
{
    using CB = CombineBatch<D, G>;
    constexpr int CPL = CB::CPL, NB = CB::NB, PR = part_rec<D>();
    const int jm = lane % NB, hm = lane / NB;
    const bool mine = hm < G && k0 + jm < team;
    const uint32_t pm = ub + (uint32_t)(k0 + (mine ? jm : 0)) * stride + (uint32_t)(mine ? hm : 0) * PR * 4u;
    b.m = mine ? load_shared(r, pm) : -__builtin_inff();
    b.l = mine ? load_shared(r, pm + 4u) : 0.0f;
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int j = 0; j < NB; j++)
#pragma unroll
            for (int s = 0; s < CPL; s++)
                b.o[h][j][s] = k0 + j < team ? load_shared(r, ub + (uint32_t)(k0 + j) * stride +
                                                                  ((uint32_t)h * PR + 4u + lane + 64u * s) * 4u)
                                             : 0.0f;
}

// Fold `count` partial states (slots first, first + step, ... in units of records) into the
// state (M, L, O), which holds the sink state or an empty one on entry.
template <int D, int G>
__device__ __forceinline__ void fold_states(const DecodeParams &p, int first, int step, int count, int lane,
                                            float (&M)[G], float (&L)[G], float (&O)[G][D / 64])
{
    using CB = CombineBatch<D, G>;
    constexpr int CPL = CB::CPL, NB = CB::NB, PR = part_rec<D>();
    const uint32_t stride = (uint32_t)step * G * PR * 4u; // bytes between the states
    // all slots are below the number of waves
    const rsrc_t r = make_rsrc(p.part, (uint32_t)p.n_waves * G * PR * 4u);
    const uint32_t ub = (uint32_t)first * G * PR * 4u;    // first state, head 0
    CB cur, nxt;
    load_batch<D, G>(cur, r, ub, stride, 0, count, lane);
    for (int k0 = 0; k0 < count; k0 += NB) {
        if (k0 + NB < count)
            load_batch<D, G>(nxt, r, ub, stride, k0 + NB, count, lane);
#pragma unroll
        for (int h = 0; h < G; h++) {
#pragma unroll
            for (int j = 0; j < NB; j++) {
                const float mj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cur.m), h * NB + j));
                const float lj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cur.l), h * NB + j));
                if (mj == -__builtin_inff())
                    continue;
                const float Mn = fmaxf(M[h], mj);
                const float fo = M[h] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(M[h] - Mn);
                const float fn = __builtin_amdgcn_exp2f(mj - Mn);
                L[h] = fmaf(L[h], fo, lj * fn);
#pragma unroll
                for (int s = 0; s < CPL; s++)
                    O[h][s] = fmaf(O[h][s], fo, cur.o[h][j][s] * fn);
                M[h] = Mn;
            }
        }
        cur = nxt;
    }
}

// The unit's team, last step: fold `count` states (stripe or member states) into the sink
// positions' state and write the normalised output out_u[h][D].
template <int D, int G>
__device__ __forceinline__ void combine_unit(const DecodeParams &p, const float *sink, int first, int step, int count,
                                             int lane, float *out_u)
{
    constexpr int CPL = D / 64;
    float M[G], L[G], O[G][CPL];
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float *sk = sink + h * (D + 2);
        M[h] = sk[0];
        L[h] = sk[1];
#pragma unroll
        for (int s = 0; s < CPL; s++)
            O[h][s] = sk[2 + lane + 64 * s];
    }
    fold_states<D, G>(p, first, step, count, lane, M, L, O);
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int s = 0; s < CPL; s++)
            out_u[h * D + lane + 64 * s] = L[h] > 0.0f ? O[h][s] / L[h] : 0.0f;
}

// A stripe's last member: fold the stripe's member states into one state, stored (not
// normalised) in the slot of the stripe's first member.
template <int D, int G>
__device__ __forceinline__ void combine_stripe(const DecodeParams &p, int first, int step, int count, int lane)
{
    constexpr int CPL = D / 64, PR = part_rec<D>();
    float M[G], L[G], O[G][CPL];
#pragma unroll
    for (int h = 0; h < G; h++) {
        M[h] = -__builtin_inff();
        L[h] = 0.0f;
#pragma unroll
        for (int s = 0; s < CPL; s++)
            O[h][s] = 0.0f;
    }
    fold_states<D, G>(p, first, step, count, lane, M, L, O);
    const rsrc_t r = make_rsrc(p.part, (uint32_t)p.n_waves * G * PR * 4u);
#pragma unroll
    for (int h = 0; h < G; h++) {
        const uint32_t rb = ((uint32_t)first * G + h) * PR * 4u;
        if (lane == 0)
            store_shared2(r, rb, M[h], L[h]);
#pragma unroll
        for (int s = 0; s < CPL; s++)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[h][s]), r, rb + (4u + lane + 64u * s) * 4u, 0,
                                                  kCoherent);
    }
}

// Register budget: 4 heads over INT2 or Lloyd-Max keys fit 3 waves per SIMD (168 VGPRs);
// asymmetric 4-bit keys (twice the key words and their scales in flight) and 8 heads get 2.
//
// Work split: the grid holds one wave per resident slot of the device, at least one per unit
// (see team_size).  Waves resident on one SIMD get unequal shares of its issue slots (older
// waves first), so tiles are handed out at run time: a unit's team draws them from a
// per-unit counter that the query-prep kernel zeroes.  A unit served by one wave gets its
// normalised output from it; otherwise each member writes one partial softmax state
// (m, l, o) in the slot of its place, and the last member to finish combines them.
// Unnormalised Walsh-Hadamard transform of D values held 8 per lane by lanes 0 .. D/8 - 1
// (lane l: values 8l .. 8l + 7): in-lane stages, then xor shuffles between lanes.  Every lane
// of the wave takes part (lanes past D/8 exchange among themselves only).
template <int D>
__device__ __forceinline__ void fwht8_lanes(float (&v)[8], int lane)
{
#pragma unroll
    for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
        for (int j = 0; j < 8; j++)
            if ((j & hs) == 0) {
                const float a = v[j], b = v[j + hs];
                v[j] = a + b;
                v[j + hs] = a - b;
            }
#pragma unroll
    for (int m = 1; m < D / 8; m <<= 1)
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float other = __shfl_xor(v[j], m);
            v[j] = (lane & m) ? other - v[j] : v[j] + other;
        }
}

// KQV values: the weighted sums over a wave's positions, in the rotated coordinates, are
// A = sum_t p_t rho_t cent[code_t] (o on entry) and, per channel, the sketch-bit sums
// b_j = sum_t p_t gamma_t bit_t (scaled by the halves' place values) with g = sum_t p_t gamma_t.
// The QJL estimator and the inverse rotation are linear, so they apply once here:
//   o = FWHT(A + sqrt(pi/2)/D * D_qjl FWHT(g - 2 b)) / D.
template <int D>
__device__ __forceinline__ void kqv_out(float (&o)[8], const float (&b)[8], float g, int lane, const uint32_t *qjl)
{
    constexpr int LPP = D / 8;
    float h[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const float place = (j & 3) == 0 ? 2097152.0f : (j & 3) == 1 ? 131072.0f : 8192.0f; // 2^21, 2^17, 2^13
        h[j] = lane < LPP ? g - 2.0f * (b[j] * place) : 0.0f;
    }
    fwht8_lanes<D>(h, lane);
    const float c = 1.2533141373155003f / (float)D; // sqrt(pi / 2) / D
    const uint32_t sw = lane < LPP ? qjl[lane / 4] >> (8 * (lane % 4)) : 0u; // this lane's 8 sign bits
#pragma unroll
    for (int j = 0; j < 8; j++)
        o[j] = fmaf(c, ((sw >> j) & 1u) ? -h[j] : h[j], lane < LPP ? o[j] : 0.0f);
    fwht8_lanes<D>(o, lane);
#pragma unroll
    for (int j = 0; j < 8; j++)
        o[j] *= 1.0f / (float)D;
}

template <int D, int G, int KF, int VF>
__global__ __launch_bounds__(kWave)
// (KQV values keep a second set of per-channel sums: fewer waves, no spills)
__attribute__((amdgpu_waves_per_eu(VF == KVQ_V_KQV ? (G <= 2 ? 3 : G == 4 ? 2 : 1)
                                                   : (G < 4 || (G == 4 && KF != KVQ_K_ASYM4)) ? 3 : 2)))
void decode_kernel(DecodeParams p, const uint32_t *__restrict__ qrec)
{
    using C = Cfg<D, G, KF, VF>;
    constexpr int KROWS = C::KROWS, NGV = C::NGV, NP = C::NP;
    constexpr int TPL = C::TPL, TILE = C::TILE, WPP = C::WPP, LPP = C::LPP, PPI = C::PPI;
    constexpr int VIT = C::VIT, VW = C::VW, WV = C::WV;
    constexpr bool V2 = VF == KVQ_V_ASYM2_TOKEN; // per-token INT2 values
    constexpr bool KQ = VF == KVQ_V_KQV;         // KQV values (3-bit codes + sketch bits)
    using VWord = std::conditional_t<V2, uint32_t, uint2>; // a lane's value words of one pair
    __shared__ Smem<D, G, KF, VF> sm;

    const int lane = threadIdx.x;
    const int w = blockIdx.x;
    const int Tu = p.tiles_per_unit;
    const int x = sgpr(team_slot(w, p.n_waves, p.n_cu));       // this wave's place
    const int u = sgpr(x % p.n_units);                          // its unit
    const int team = sgpr(team_size(u, p.n_units, p.n_waves)); // waves serving it
    const int n_q_heads = p.n_kv_heads * G;
    const uint32_t ucap = (uint32_t)p.cap;

    if constexpr (KF == KVQ_K_LLOYD4) {
        // code-pair table: byte (lo nibble a, hi nibble b) -> fp16 (cent[a], cent[b])
        for (int e = lane; e < 256; e += kWave)
            sm.lut[e] = pack_f16x2(p.codebook[e & 15], p.codebook[e >> 4]);
        __syncthreads();
    }
    if constexpr (KQ) {
        // byte (code nibbles of two channels of one position) -> fp16 centroid pair
        for (int e = lane; e < 256; e += kWave)
            sm.vlut[e] = pack_f16x2(p.v_codebook[e & 7], p.v_codebook[(e >> 4) & 7]);
        __syncthreads();
    }

    const int vs = lane % LPP;         // value slot: channels 8*vs .. 8*vs+7
    const int vgrp = (V2 || KQ) ? 0 : vs / 4;  // its scale group (one per token for INT2 and KQV)
    const uint32_t vvo = ((uint32_t)(lane / LPP) * WPP + (uint32_t)(VW * vs)) * 4u; // value word offset
    const int q_lo = p.n_sink, q_hi = p.q_end; // quantized positions [q_lo, q_hi)

    // ---- the unit's query scalars (uniform loads from its record).  Under bucket-relative
    // RoPE every bucket of w positions has a record of its own (query rotated back by the
    // bucket's anchor, its mask and scales): tile t reads record t >> tlw; without RoPE
    // tlw = 31, so every tile reads the first one.  The first record also holds the BF16
    // positions' softmax state.
    const uint32_t *__restrict__ rec = qrec + (size_t)u * p.n_rb * C::QREC;
    const int tlw = p.rope_lw ? p.rope_lw - 7 : 31; // log2 of the tiles per bucket
    static_assert(C::TILE == 1 << 7, "tiles per bucket");
    const uint32_t mask = rec[C::OFF_MASK];
    float acc_to_logit[G], logit_to_acc[G];
    int qbk = 0; // bucket whose scales acc_to_logit / logit_to_acc hold
    auto load_scales = [&](int bq) {
        const float *recf = reinterpret_cast<const float *>(rec + (size_t)bq * C::QREC);
#pragma unroll
        for (int h = 0; h < G; h++) {
            acc_to_logit[h] = recf[C::OFF_QSC + h];
            logit_to_acc[h] = 1.0f / acc_to_logit[h];
        }
    };
    load_scales(0);

    // ---- running softmax state of the current unit
    float acc[G][8];
    float bacc[G][KQ ? 8 : 1]; // KQV: sketch-bit sums per channel
    float zacc[G][NGV];
    float lsum[G];
    float mrun[G], mthr[G];
    auto reset = [&]() {
#pragma unroll
        for (int h = 0; h < G; h++) {
            lsum[h] = 0.0f;
            mrun[h] = -__builtin_inff();
            mthr[h] = -__builtin_inff();
#pragma unroll
            for (int j = 0; j < 8; j++)
                acc[h][j] = 0.0f;
#pragma unroll
            for (int g = 0; g < NGV; g++)
                zacc[h][g] = 0.0f;
#pragma unroll
            for (int j = 0; j < (KQ ? 8 : 1); j++)
                bacc[h][j] = 0.0f;
        }
    };

    // stripes: a team of more than kStripe waves splits into S stripes of B = ceil(team / S)
    // consecutive members (the last one may have fewer); a stripe serves a contiguous range
    // of the unit's tiles in proportion to its members, with a counter of its own at the
    // place of its first member, so no counter takes more than kStripe waves' draws.
    // Consecutive members sit at different ages on their compute units (see team_slot), so
    // every stripe gets a mix of fast and slow waves and the stripes end together.
    const int member = sgpr(x / p.n_units);
    const int S = sgpr((team + kStripe - 1) / kStripe);
    const int B = sgpr((team + S - 1) / S);
    const int stripe = sgpr(member / B);
    const int m0 = stripe * B;                                 // its first member
    const int smem = sgpr(member - m0);                        // index within the stripe
    const int nst = sgpr(min(m0 + B, team) - m0);              // members of the stripe
    const int ts0 = sgpr((int)((long long)m0 * Tu / team));    // its tiles [ts0, ts1)
    const int ts1 = sgpr((int)((long long)(m0 + nst) * Tu / team));

    // ---- end of this wave's tiles: reduce over the wave, then write the normalised output
    // (the unit's only wave) or this wave's partial state
    auto flush = [&]() {
        const bool whole = team == 1;
        const int b = u / p.n_kv_heads;
        const int kvh = u % p.n_kv_heads;
        float4 *red = sm.red; // the weight buffer is free at the end of the tiles
#pragma unroll
        for (int h = 0; h < G; h++) {
            // lanes vs, vs + LPP, ... hold partial sums of the same 8 channels: add them
            // through LDS (the weight buffer is free here)
            red[2 * lane] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
            red[2 * lane + 1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
            __syncthreads();
            const float ls = wave_sum_dpp(lsum[h]);
            float zs[NGV];
#pragma unroll
            for (int g = 0; g < NGV; g++)
                zs[g] = wave_sum_dpp(zacc[h][g]);
            float o[8] = {acc[h][0], acc[h][1], acc[h][2], acc[h][3], acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
            if (lane < LPP) {
#pragma unroll
                for (int k = 1; k < 64 / LPP; k++) {
                    const float4 a0 = red[2 * (lane + k * LPP)], a1 = red[2 * (lane + k * LPP) + 1];
                    o[0] += a0.x; o[1] += a0.y; o[2] += a0.z; o[3] += a0.w;
                    o[4] += a1.x; o[5] += a1.y; o[6] += a1.z; o[7] += a1.w;
                }
            }
            if constexpr (KQ) {
                // the sketch-bit sums, reduced the same way, then the estimator and the
                // inverse rotation (every lane takes part in the shuffles)
                __syncthreads();
                red[2 * lane] = make_float4(bacc[h][0], bacc[h][1], bacc[h][2], bacc[h][3]);
                red[2 * lane + 1] = make_float4(bacc[h][4], bacc[h][5], bacc[h][6], bacc[h][7]);
                __syncthreads();
                float bs[8] = {bacc[h][0], bacc[h][1], bacc[h][2], bacc[h][3],
                               bacc[h][4], bacc[h][5], bacc[h][6], bacc[h][7]};
                if (lane < LPP) {
#pragma unroll
                    for (int k = 1; k < 64 / LPP; k++) {
                        const float4 a0 = red[2 * (lane + k * LPP)], a1 = red[2 * (lane + k * LPP) + 1];
                        bs[0] += a0.x; bs[1] += a0.y; bs[2] += a0.z; bs[3] += a0.w;
                        bs[4] += a1.x; bs[5] += a1.y; bs[6] += a1.z; bs[7] += a1.w;
                    }
                }
                kqv_out<D>(o, bs, zs[0], lane, p.v_qjl);
            }
            if (lane < LPP) {
                if constexpr (!KQ) {
                // INT4: even slots summed code_even + 16 code_odd, odd slots 16 code_odd.
                // INT2: slots 4k..4k+3 summed c0 + 4 c1, 4 c1, 16 c2 + 64 c3, 64 c3.  Either
                // way an even slot takes out the next slot's sums, and the scales undo the
                // codes' places in the subnormal halves.
#pragma unroll
                for (int j = 0; j < 8; j += 2)
                    o[j] -= o[j + 1];
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    float sc;
                    if constexpr (V2)
                        sc = (j & 3) == 0 ? 16777216.0f : (j & 3) == 1 ? 4194304.0f : (j & 3) == 2 ? 1048576.0f : 262144.0f;
                    else
                        sc = (j & 1) ? 1048576.0f : 16777216.0f; // undo 2^-20 / 2^-24
                    o[j] = o[j] * sc + zs[V2 ? 0 : (8 * lane + j) / 32];
                }
                }
                if (whole) {
                    // fold in the sink positions' state, then normalise
                    const float *sk = reinterpret_cast<const float *>(rec) + C::OFF_SINK + h * (D + 2);
                    const float ms = sk[0];
                    const float M = fmaxf(mrun[h], ms);
                    const float fw = mrun[h] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mrun[h] - M);
                    const float fs = ms == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
                    const float L = fmaf(ls, fw, sk[1] * fs);
                    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
                    for (int j = 0; j < 8; j++)
                        o[j] = fmaf(o[j], fw, sk[2 + 8 * lane + j] * fs) * inv;
                    float4 *dst = reinterpret_cast<float4 *>(p.out + ((size_t)b * n_q_heads + (size_t)kvh * G + h) * D + 8 * lane);
                    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
                    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
                } else {
                    const rsrc_t pr = make_rsrc(p.part, (uint32_t)p.n_waves * G * part_rec<D>() * 4u);
                    const uint32_t rb = ((uint32_t)x * G + h) * part_rec<D>() * 4u;
                    if (lane == 0)
                        store_shared2(pr, rb, mrun[h], ls);
                    store_shared4(pr, rb + (4u + 8u * lane) * 4u, o[0], o[1], o[2], o[3]);
                    store_shared4(pr, rb + (8u + 8u * lane) * 4u, o[4], o[5], o[6], o[7]);
                }
            }
            __syncthreads();
        }
        if (!whole) {
            // count this member in once its states are stored (all of the wave's memory
            // operations complete); the member that arrives last combines the states (in
            // member order, so the result does not depend on which member that is) with the
            // sink positions' state.  A striped team does it in two steps: the last member of
            // each stripe folds the stripe's states into its first member's slot and then
            // counts the stripe in; the last stripe folds the stripes' states.
            const float *sink = reinterpret_cast<const float *>(rec) + C::OFF_SINK;
            float *out_u = p.out + ((size_t)b * n_q_heads + (size_t)kvh * G) * D;
            __builtin_amdgcn_s_waitcnt(0);
            uint32_t arrived = 0;
            if (S == 1) {
                if (lane == 0)
                    arrived = __hip_atomic_fetch_add(p.tile_ctr + 2 * p.n_waves + u, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                if ((int)uniform(arrived) == team - 1)
                    combine_unit<D, G>(p, sink, u, p.n_units, team, lane, out_u);
            } else {
                const int sfirst = u + m0 * p.n_units; // place of the stripe's first member
                if (lane == 0)
                    arrived = __hip_atomic_fetch_add(p.tile_ctr + p.n_waves + sfirst, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                if ((int)uniform(arrived) == nst - 1) {
                    combine_stripe<D, G>(p, sfirst, p.n_units, nst, lane);
                    __builtin_amdgcn_s_waitcnt(0);
                    uint32_t done = 0;
                    if (lane == 0)
                        done = __hip_atomic_fetch_add(p.tile_ctr + 2 * p.n_waves + u, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
                    if ((int)uniform(done) == S - 1)
                        combine_unit<D, G>(p, sink, u, B * p.n_units, S, lane, out_u);
                }
            }
        }
    };

    // this wave's tiles: tile `member` first, then those the unit's counter hands out.  The
    // counter is asked one tile ahead of the answer's use (lane 0's atomic; its return
    // travels with the tile loads), so the next tile's loads can still go out a whole tile
    // before its scoring: key-side words and value words of the current tile are in
    // registers, and value word pair `it` is reloaded with the next tile's right after its
    // last use.
    KTile<D, G, KF, VF> cur;
    VWord vcur[VIT];
    reset();
    const Slabs sl = unit_slabs<D, G, KF, VF>(p, u);
    uint32_t *const ctr = p.tile_ctr + (u + m0 * p.n_units);
    const bool dynamic = p.dynamic && nst > 1;
    uint32_t ask = 0;
    if (dynamic && lane == 0)
        ask = draw_tile(ctr);
    // the tile loop, compiled for every-row-kept or not (ALL) and channel 0 apart or not
    // (CH0), so that neither costs a branch per tile
    auto tiles = [&](auto all_c, auto ch0_c, auto rope_c) {
        constexpr bool ALL = decltype(all_c)::value;
        constexpr bool CH0 = decltype(ch0_c)::value;
        constexpr bool RP = decltype(rope_c)::value; // per-bucket records (bucket-relative RoPE)
        // mask of the tile in `cur` (its bucket's; without RoPE the unit's)
        uint32_t mcur = mask;
        {
            const int t = ts0 + smem;
            const uint32_t off = t < ts1 ? 0u : kNoAccess;
            if (RP && t < ts1)
                mcur = rec[(size_t)(t >> tlw) * C::QREC + C::OFF_MASK];
            load_ktile<D, G, KF, VF, ALL, CH0>(cur, sl, ucap, lane, t * TILE, mcur, off);
#pragma unroll
            for (int it = 0; it < VIT; it++)
                vcur[it] = vload<V2>(sl.vc, vvo + off, ((uint32_t)(t * TILE / 2 + it * PPI) * WPP) * 4u);
        }
        for (int t = ts0 + smem; t < ts1;) {
            const int t0 = t * TILE;
            const int tl = t0 + lane * TPL;
            const int tn = dynamic ? ts0 + nst + (int)uniform(ask) : t + nst; // the tile after this one
            const bool more = tn < ts1;
            if (dynamic && more && lane == 0)
                ask = draw_tile(ctr);
            set_priority_for(t - ts0, ts1 - ts0);

            // ---- scores (accumulator units; log2 logit = lg * acc_to_logit[h]).  The query
            // operands are read through an address that depends on the tile number (the
            // added term is always 0: t >= 0), so they are reloaded per tile from the scalar
            // cache rather than hoisted out of the loop into more scalar registers than exist.
            const int bt = RP ? t >> tlw : 0;
            const uint32_t *__restrict__ rq = rec + ((uint32_t)t >> 31) + (size_t)bt * C::QREC;
            if (RP && bt != qbk) {
                // a tile of another bucket: its scales, and the raise threshold in its units
                load_scales(bt);
                qbk = bt;
#pragma unroll
                for (int h = 0; h < G; h++)
                    mthr[h] = (mrun[h] + kSlack) * logit_to_acc[h];
            }
            float lg[TPL][G];
#pragma unroll
            for (int i = 0; i < TPL; i++)
#pragma unroll
                for (int h = 0; h < G; h++)
                    lg[i][h] = 0.0f;
            if constexpr (KF != KVQ_K_LLOYD4) {
                score_asym<D, G, KF, VF, ALL, CH0>(cur, rq, mcur, lg);
            } else {
#pragma unroll
                for (int r = 0; r < KROWS; r++) {
                    if (!ALL && !(mcur >> (r / C::RPP) & 1u))
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
                            const uint32_t qv = rq[C::OFF_QP + (r * G + h) * C::QW + j];
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
            uint32_t vsw[TPL][NGV];
#pragma unroll
            for (int gg = 0; gg < NGV; gg++) {
                vsw[0][gg] = cur.vsz[gg].x;
                vsw[1][gg] = cur.vsz[gg].y;
            }
            const bool full = (t0 >= q_lo) && (t0 + TILE <= q_hi);
            if (!full) {
#pragma unroll
                for (int i = 0; i < TPL; i++) {
                    const int tp = tl + i;
                    if (tp < q_lo || tp >= q_hi) {
#pragma unroll
                        for (int h = 0; h < G; h++)
                            lg[i][h] = -__builtin_inff();
#pragma unroll
                        for (int gg = 0; gg < NGV; gg++)
                            vsw[i][gg] = 0u;
                    }
                }
            }

            // ---- next tile's key-side words, into the registers this tile no longer needs:
            // in flight during the rest of this tile.  After the wave's last tile the loads
            // access nothing.
            const uint32_t noff = more ? 0u : kNoAccess;
            if constexpr (RP)
                mcur = more ? rec[(size_t)(tn >> tlw) * C::QREC + C::OFF_MASK] : mask;
            load_ktile<D, G, KF, VF, ALL, CH0>(cur, sl, ucap, lane, tn * TILE, mcur, noff);

            // ---- online softmax (log2 units), per head.  The running maximum m is raised
            // (wave-wide DPP max, rescale of that head's state) only when a logit exceeds
            // m + kSlack; otherwise weights 2^(l - m) may reach 2^kSlack, which keeps every
            // fp16 weight p*s finite (s < 2^14 for inputs below 65504) and makes the raise
            // rare after the first tile.  The test runs in accumulator units against
            // mthr = (m + kSlack) / acc_to_logit; a rounding miss is harmless.
            // One branch per tile covers all heads: one per head splits the tile's code into
            // blocks the compiler cannot schedule across, which costs far more than the
            // raises themselves (about one per two tiles over all heads).
            uint64_t above[G];
            uint64_t any_above = 0;
#pragma unroll
            for (int h = 0; h < G; h++) {
                above[h] = 0;
#pragma unroll
                for (int i = 0; i < TPL; i++)
                    above[h] |= __ballot(lg[i][h] > mthr[h]);
                any_above |= above[h];
            }
            if (any_above) {
#pragma unroll
                for (int h = 0; h < G; h++) {
                    if (!above[h])
                        continue;
                    float mt = lg[0][h];
#pragma unroll
                    for (int i = 1; i < TPL; i++)
                        mt = fmaxf(mt, lg[i][h]);
                    const float mnew = fmaxf(mrun[h], wave_max_dpp(mt * acc_to_logit[h]));
                    const float alpha = __builtin_amdgcn_exp2f(mrun[h] - mnew);
                    mrun[h] = mnew;
                    mthr[h] = (mnew + kSlack) * logit_to_acc[h];
                    lsum[h] *= alpha;
#pragma unroll
                    for (int j = 0; j < 8; j++)
                        acc[h][j] *= alpha;
#pragma unroll
                    for (int gg = 0; gg < NGV; gg++)
                        zacc[h][gg] *= alpha;
                    if constexpr (KQ) {
#pragma unroll
                        for (int j = 0; j < 8; j++)
                            bacc[h][j] *= alpha;
                    }
                }
            }
            // (a running maximum still at -inf means every logit so far, this tile's included,
            // is -inf: subtract 0 instead so the weights come out 0, not NaN)
            float pw[TPL][G];
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float msub = mrun[h] == -__builtin_inff() ? 0.0f : mrun[h];
#pragma unroll
                for (int i = 0; i < TPL; i++)
                    pw[i][h] = __builtin_amdgcn_exp2f(fmaf(lg[i][h], acc_to_logit[h], -msub));
            }
            // zero-point term and the fp16 weights p*s of this lane's position pair (-> LDS),
            // from the weights rounded to fp16 pairs: one packed product and one dot2 per
            // (group, head)
            // (the softmax sum takes the same fp16-rounded weights the values get: one dot2)
            uint32_t ph[G];
#pragma unroll
            for (int h = 0; h < G; h++) {
                ph[h] = pack_f16x2(pw[0][h], pw[1][h]);
                lsum[h] = dot2(ph[h], 0x3C003C00u, lsum[h]); // (1.0, 1.0)
            }
#pragma unroll
            for (int gg = 0; gg < NGV; gg++) {
                const uint32_t sp = __builtin_amdgcn_perm(vsw[1][gg], vsw[0][gg], 0x05040100u); // (s0, s1)
                const uint32_t zp = __builtin_amdgcn_perm(vsw[1][gg], vsw[0][gg], 0x07060302u); // (z0, z1)
                uint32_t wq[4 * WV];
#pragma unroll
                for (int h = 0; h < G; h++) {
                    zacc[h][gg] = dot2(ph[h], zp, zacc[h][gg]);
                    wq[h] = mul_f16x2(ph[h], sp);
                }
#pragma unroll
                for (int h = G; h < 4 * WV; h++)
                    wq[h] = 0u;
#pragma unroll
                for (int v4 = 0; v4 < WV; v4++)
                    sm.w[gg][lane][v4] = make_uint4(wq[4 * v4], wq[4 * v4 + 1], wq[4 * v4 + 2], wq[4 * v4 + 3]);
                if constexpr (KQ) {
                    // KQV: the second weight set, p * (residual norm), for the sketch bits
#pragma unroll
                    for (int h = 0; h < G; h++)
                        wq[h] = mul_f16x2(ph[h], zp);
#pragma unroll
                    for (int v4 = 0; v4 < WV; v4++)
                        sm.w[1][lane][v4] = make_uint4(wq[4 * v4], wq[4 * v4 + 1], wq[4 * v4 + 2], wq[4 * v4 + 3]);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            // ---- values: lane owns channels 8*vs .. 8*vs+7 of one pair per iteration
            const uint32_t vnext = (uint32_t)(tn * TILE / 2) * WPP * 4u;
#pragma unroll
            for (int it = 0; it < VIT; it++) {
                const VWord vv = vcur[it];
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
                if constexpr (KQ) {
                    // KQV: nibble k of each half = 3-bit code | sketch bit << 3 of channel
                    // 8*vs + 4*q2 + k.  Centroid pairs of the two positions from the LDS table;
                    // the sketch bits masked in place are exact fp16 halves 2^-21, 2^-17, 2^-13
                    // (nibble 3 moved down by 4 bits) summed with the p * gamma weights.
                    uint32_t wb[4 * WV];
#pragma unroll
                    for (int v4 = 0; v4 < WV; v4++) {
                        const uint4 t4 = sm.w[1][pl][v4];
                        wb[4 * v4 + 0] = t4.x;
                        wb[4 * v4 + 1] = t4.y;
                        wb[4 * v4 + 2] = t4.z;
                        wb[4 * v4 + 3] = t4.w;
                    }
#pragma unroll
                    for (int q2 = 0; q2 < 2; q2++) {
                        const uint32_t x = q2 == 0 ? vv.x : vv.y;
                        // a byte holds two channels of one position: its table entry is their
                        // centroid pair; two permutes regroup the entries by channel across the
                        // position pair
                        const uint32_t r0 = sm.vlut[x & 0xFFu], r1 = sm.vlut[(x >> 8) & 0xFFu];
                        const uint32_t r2 = sm.vlut[(x >> 16) & 0xFFu], r3 = sm.vlut[x >> 24];
                        const uint32_t cp[4] = {__builtin_amdgcn_perm(r2, r0, 0x05040100u),
                                                __builtin_amdgcn_perm(r2, r0, 0x07060302u),
                                                __builtin_amdgcn_perm(r3, r1, 0x05040100u),
                                                __builtin_amdgcn_perm(r3, r1, 0x07060302u)};
                        const uint32_t sb[4] = {x & 0x00080008u, x & 0x00800080u, x & 0x08000800u,
                                                (x >> 4) & 0x08000800u};
#pragma unroll
                        for (int h = 0; h < G; h++)
#pragma unroll
                            for (int k = 0; k < 4; k++) {
                                acc[h][4 * q2 + k] = dot2(cp[k], wv[h], acc[h][4 * q2 + k]);
                                bacc[h][4 * q2 + k] = dot2(sb[k], wb[h], bacc[h][4 * q2 + k]);
                            }
                    }
                } else if constexpr (V2) {
                    // per-token INT2: the word holds channels 8*vs .. +7 of both positions
                    // (halves), 4 two-bit codes per byte.  c0 = x & 0x000F000F is code0 +
                    // 4 code1, c1 = 4 code1, c2 = 16 code2 + 64 code3, c3 = 64 code3 (all
                    // subnormal halves); bytes 1 and 3 likewise after one byte permute.
                    const uint32_t x = vv;
                    const uint32_t y = __builtin_amdgcn_perm(0u, x, 0x0c030c01u); // bytes 1, 3 -> 0, 2
                    const uint32_t c[8] = {x & 0x000F000Fu, x & 0x000C000Cu, x & 0x00F000F0u, x & 0x00C000C0u,
                                           y & 0x000F000Fu, y & 0x000C000Cu, y & 0x00F000F0u, y & 0x00C000C0u};
#pragma unroll
                    for (int h = 0; h < G; h++)
#pragma unroll
                        for (int j = 0; j < 8; j++)
                            acc[h][j] = dot2(c[j], wv[h], acc[h][j]);
                } else {
#pragma unroll
                for (int q2 = 0; q2 < 2; q2++) {
                    // c0 holds both nibbles of bytes 0 and 2 (code0 + 16 code1, still a
                    // subnormal half), c1 code1 alone; the flush subtracts c1's sums from c0's.
                    // Bytes 1 and 3 likewise, moved down by one byte permute.
                    const uint32_t x = q2 == 0 ? vv.x : vv.y;
                    const uint32_t y = __builtin_amdgcn_perm(0u, x, 0x0c030c01u); // bytes 1, 3 -> 0, 2
                    const uint32_t c0 = x & 0x00FF00FFu, c1 = x & 0x00F000F0u;
                    const uint32_t c2 = y, c3 = y & 0x00F000F0u;
#pragma unroll
                    for (int h = 0; h < G; h++) {
                        acc[h][4 * q2 + 0] = dot2(c0, wv[h], acc[h][4 * q2 + 0]);
                        acc[h][4 * q2 + 1] = dot2(c1, wv[h], acc[h][4 * q2 + 1]);
                        acc[h][4 * q2 + 2] = dot2(c2, wv[h], acc[h][4 * q2 + 2]);
                        acc[h][4 * q2 + 3] = dot2(c3, wv[h], acc[h][4 * q2 + 3]);
                    }
                }
                }
                // reload after the last use, into the same registers
                vcur[it] = vload<V2>(sl.vc, vvo + noff, vnext + (uint32_t)(it * PPI * WPP) * 4u);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            t = tn;
        }
    };
    // (bucket-relative RoPE takes the pruned-rows variant whatever the masks: they differ
    // by bucket)
    if (p.rope_lw) {
        if (KF != KVQ_K_LLOYD4 && p.ch0)
            tiles(BoolC<false>(), BoolC<KF != KVQ_K_LLOYD4>(), BoolC<true>());
        else
            tiles(BoolC<false>(), BoolC<false>(), BoolC<true>());
    } else if (mask == (1u << NP) - 1u) {
        if (KF != KVQ_K_LLOYD4 && p.ch0)
            tiles(BoolC<true>(), BoolC<KF != KVQ_K_LLOYD4>(), BoolC<false>());
        else
            tiles(BoolC<true>(), BoolC<false>(), BoolC<false>());
    } else {
        if (KF != KVQ_K_LLOYD4 && p.ch0)
            tiles(BoolC<false>(), BoolC<KF != KVQ_K_LLOYD4>(), BoolC<false>());
        else
            tiles(BoolC<false>(), BoolC<false>(), BoolC<false>());
    }
    flush();
}

// ===================================================================== launchers
template <int D, int G, int KF, int VF>
hipError_t launch_one(int units, const DecodeParams &p, hipEvent_t const ev[2], hipStream_t s)
{
    if (p.n_sink > 8)
        hipLaunchKernelGGL((qprep_kernel<D, G, KF, 32>), dim3((unsigned)(p.n_qb * units)), dim3(kWave * G), 0, s, p);
    else
        hipLaunchKernelGGL((qprep_kernel<D, G, KF, 8>), dim3((unsigned)(p.n_qb * units)), dim3(kWave * G), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (ev[0] && (e = hipEventRecord(ev[0], s)) != hipSuccess)
        return e;
    hipLaunchKernelGGL((decode_kernel<D, G, KF, VF>), dim3((unsigned)p.n_waves), dim3(kWave), 0, s, p,
                       static_cast<const uint32_t *>(p.qprep));
    e = hipGetLastError();
    if (e == hipSuccess && ev[1])
        e = hipEventRecord(ev[1], s);
    return e;
}

template <int D, int G, int VF>
hipError_t launch_kf(int kfmt, int units, const DecodeParams &p, hipEvent_t const ev[2], hipStream_t s)
{
    switch (kfmt) {
    case KVQ_K_ASYM2: return launch_one<D, G, KVQ_K_ASYM2, VF>(units, p, ev, s);
    case KVQ_K_ASYM4: return launch_one<D, G, KVQ_K_ASYM4, VF>(units, p, ev, s);
    default: return launch_one<D, G, KVQ_K_LLOYD4, VF>(units, p, ev, s);
    }
}

template <int D, int VF>
hipError_t launch_g(int group, int kfmt, int units, const DecodeParams &p, hipEvent_t const ev[2],
                    hipStream_t s)
{
    switch (group) {
    case 1: return launch_kf<D, 1, VF>(kfmt, units, p, ev, s);
    case 2: return launch_kf<D, 2, VF>(kfmt, units, p, ev, s);
    case 4: return launch_kf<D, 4, VF>(kfmt, units, p, ev, s);
    default: return launch_kf<D, 8, VF>(kfmt, units, p, ev, s);
    }
}

template <int VF>
hipError_t launch_vf(int head_dim, int group, int kfmt, int units, const DecodeParams &p, hipEvent_t const ev[2],
                     hipStream_t s)
{
    if (head_dim == 128)
        return launch_g<128, VF>(group, kfmt, units, p, ev, s);
    return launch_g<64, VF>(group, kfmt, units, p, ev, s);
}

template <int D, int G, int KF, int VF>
const void *kernel_of() { return reinterpret_cast<const void *>(&decode_kernel<D, G, KF, VF>); }

template <int D, int G, int VF>
const void *kernel_kf(int kfmt)
{
    return kfmt == KVQ_K_ASYM2 ? kernel_of<D, G, KVQ_K_ASYM2, VF>()
           : kfmt == KVQ_K_ASYM4 ? kernel_of<D, G, KVQ_K_ASYM4, VF>()
                                 : kernel_of<D, G, KVQ_K_LLOYD4, VF>();
}

template <int D, int VF>
const void *kernel_g(int group, int kfmt)
{
    return group == 1 ? kernel_kf<D, 1, VF>(kfmt) : group == 2 ? kernel_kf<D, 2, VF>(kfmt)
           : group == 4 ? kernel_kf<D, 4, VF>(kfmt) : kernel_kf<D, 8, VF>(kfmt);
}

template <int VF>
const void *kernel_vf(int head_dim, int group, int kfmt)
{
    return head_dim == 128 ? kernel_g<128, VF>(group, kfmt) : kernel_g<64, VF>(group, kfmt);
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
} // namespace kvq
