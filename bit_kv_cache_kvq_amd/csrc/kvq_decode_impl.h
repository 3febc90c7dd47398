// kvq_decode_impl.h -- decode attention scored straight from the packed low-bit cache.
// (Kernel templates; kvq_decode.hip, kvq_decode_v2.hip and kvq_decode_v3.hip instantiate them
// for the three value formats, in parallel compilations.)
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
//     its tiles and by the query prep over the BF16 positions (sinks, recent window); the
//     last wave of a unit's team to finish folds all of these states;
//   * values from INT4 codes per 32-channel group, per-token INT2 codes (Dual-QK sec. B.2),
//     or KQV's centroids and sketch bits: o = sum_t p_t s_{t,g} code_{t,c} + sum_t p_t z_{t,g}.
//
// Two kernels per decode call:
//   qprep   one wave per query head in every workgroup: per (unit, bucket) a record with the
//           mask and the fp16 query operands; per chunk of up to 64 BF16 positions (sinks,
//           recent window) the softmax state of those positions.
//   decode  one wave per resident SIMD slot (at least one per unit); the waves serving a
//           unit take its 128-position tiles in static shares, the last quarter drawn from
//           a counter.  The query record is read with uniform loads, so its operands sit in
//           scalar registers.
//           * score phase, lane per 2 positions: a key row is one dwordx2 load per lane
//             (512 B contiguous per wave).  An asymmetric code word is spread by masking
//             into registers whose fp16 halves hold one channel's code times a place factor
//             as a subnormal integer, and v_dot2_f32_f16 multiplies them with fp16 halves of
//             the query divided by the place factors: exact products, fp32 sums; a sharp
//             query adds the residual halves.  Lloyd-Max codes go through an LDS table of
//             fp16 centroid pairs and v_dot2_f32_f16 against fp16 query pairs.
//           * softmax: a running maximum per head; a wave-wide DPP reduction and a rescale
//             happen only when a tile holds a logit well above it (rare after the first
//             tiles), or when a value scale needs a lower weight exponent.
//           * value phase, lane per 8 channels: v_dot2_f32_f16 over position pairs (value
//             words interleave two positions); a code masked into the low mantissa bits of
//             a half is a subnormal integer, so no conversion is needed.  The fp16 weights
//             p*s*2^vexp of a position pair and scale group reach the value lanes through
//             LDS, all heads in one 16-byte read.
//           * the next tile's key-side words are loaded before the value phase of the
//             current one; cache reads are non-temporal (each byte is read once).
// No MFMA: this is a bandwidth-bound scan.
#pragma once

#include <atomic>
#include <type_traits>

#include <hip/hip_ext.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int D, int G, int KF, int VF = KVQ_V_ASYM4_G32>
struct Cfg {
    static constexpr int KB = (KF == KVQ_K_ASYM2) ? 2 : 4;
    static constexpr int KROWS = D * KB / 32;      // key code rows (words per position)
    static constexpr int PPW = 16 / KB;            // fp16 pairs per key word (Lloyd-Max)
    // query words per (row, head): fp16 pairs (Lloyd-Max), spread registers (asym, spread_asym)
    static constexpr int QW = (KF == KVQ_K_LLOYD4) ? 4 : (KB == 2 ? 8 : 4);
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
    // query record, u32 words per unit: mask; the sharp-query flag; per head the accumulator
    // unit (log2-logit per accumulator step) and the channel-0 coefficient; zero-term sums
    // [G][NG]; query operands [KROWS][G][QW] (fp16 halves), and their residual halves of the
    // same layout (sharp queries only)
    static constexpr int OFF_MASK = 0;
    static constexpr int OFF_SHARP = 1;
    static constexpr int OFF_QSC = 4;
    static constexpr int OFF_Q0 = OFF_QSC + G;
    static constexpr int OFF_QZ = OFF_Q0 + G;
    static constexpr int OFF_QP = (OFF_QZ + G * NG + 7) / 8 * 8;
    static constexpr int OFF_QPL = OFF_QP + KROWS * G * QW;
    static constexpr int QREC = (OFF_QPL + KROWS * G * QW + 63) / 64 * 64;
    static_assert(TILE == kTile, "host and device tile must agree");
};

// Partial softmax state record of one (wave or BF16 chunk, head): m, l, two unused words,
// o[D] (16-byte aligned).
template <int D>
constexpr int part_rec() { return D + 4; }

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
// A raised maximum is set this far (log2) above the largest logit seen, so the next raise
// waits for a logit kRaiseRoom + kSlack above it: fewer raises, at the price of weights
// 2^kRaiseRoom smaller, which raises by as much the point where small fp16 weights turn
// subnormal (they carry 2^vexp, so that point stays far below the largest weight).
constexpr float kRaiseRoom = 2.0f;
// Largest value-weight exponent (see the decode kernel): the weights 2^(l - m + vexp) stay
// below 2^(kSlack + kVexpMax) = 2^15 in fp16.
constexpr int kVexpMax = 13;
// A lowered value exponent leaves this many binades below the 2^13 bound for the largest
// scale seen, so a later, larger scale lowers it again only when it is 2^kVexpRoom times
// larger.
constexpr int kVexpRoom = 3;
// fp16 bits of the largest value scale s allowed with exponent e (s * 2^e < 2^13), in both
// halves; e = -3 allows every finite fp16 (the smallest exponent used).
__device__ __forceinline__ uint32_t vexp_thr(int e)
{
    const uint32_t b = ((uint32_t)(28 - e) << 10) - 1u;
    return b | (b << 16);
}
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// per-half unsigned maximum of two fp16 pairs (non-negative halves order as their bits)
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

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

// ===================================================================== asymmetric key spread
// A key word of an asymmetric format holds 32/KB channels of one position; its two 16-bit
// halves hold channels 0 .. 16/KB - 1 and 16/KB .. 32/KB - 1 of the word.  Spread register
// k (QW of them) keeps one field of each half in place, or after one right shift for the
// fields above bit 9, so each half is the subnormal fp16 integer P * code (value
// P * code * 2^-24, P = the field's place factor, at most 3 * 256 or 15 * 16, below 1024).
// Register k holds word-local channels (k, k + 16/KB); asym_place is P of channel c.
template <int KB>
__host__ __device__ constexpr int asym_qw() { return KB == 2 ? 8 : 4; }
template <int KB>
__device__ __forceinline__ int asym_chan(int r, int k, int hi)
{
    return r * (32 / KB) + hi * (16 / KB) + k;
}
template <int KB>
__device__ __forceinline__ float asym_place(int c)
{
    constexpr int FIELDS = 16 / KB;          // fields per half
    constexpr int DIRECT = KB == 2 ? 5 : 2;  // fields within bits 0..9 of a half
    const int j = c % FIELDS;
    return (float)(1u << (KB * (j < DIRECT ? j : j - DIRECT)));
}
template <int KB>
__device__ __forceinline__ float asym_inv_place(int c) // 1 / asym_place(c), exactly
{
    constexpr int FIELDS = 16 / KB;
    constexpr int DIRECT = KB == 2 ? 5 : 2;
    const int j = c % FIELDS;
    return __uint_as_float((uint32_t)(127 - KB * (j < DIRECT ? j : j - DIRECT)) << 23);
}
// a * b (fp16 pairs, fp32 sum) into a fresh register: the VOP3P form with an inline 0 (the
// compiler would build it from the two-address form and a v_mov of 0)
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b)
{
    float r;
    asm("v_dot2_f32_f16 %0, %2, %1, 0" : "=v"(r) : "v"(a), "s"(b));
    return r;
}
template <int KB>
__device__ __forceinline__ void spread_asym(uint32_t x, uint32_t (&o)[asym_qw<KB>()])
{
    if constexpr (KB == 2) {
        const uint32_t y = x >> 10;
#pragma unroll
        for (int k = 0; k < 5; k++)
            o[k] = x & (0x00030003u << (2 * k));
#pragma unroll
        for (int k = 5; k < 8; k++)
            o[k] = y & (0x00030003u << (2 * (k - 5)));
    } else {
        const uint32_t y = x >> 8;
        o[0] = x & 0x000F000Fu;
        o[1] = x & 0x00F000F0u;
        o[2] = y & 0x000F000Fu;
        o[3] = y & 0x00F000F0u;
    }
}

// ===================================================================== query prep
// One query record (one bucket of one unit) per workgroup, and chunks of up to 64 BF16
// positions.
// Sinks beyond this many get a workgroup of their own (else bucket 0's record workgroup
// scores them).
constexpr int kSinksInRecord = 8;

// Workgroups of the query-prep grid for a call: the window's chunks, the sinks' chunk when it
// has a workgroup of its own, then the record groups (each class unit-minor).
__host__ __device__ inline int qprep_groups(const DecodeParams &p)
{
    return (p.n_bch - 1) + (p.n_sink > kSinksInRecord ? 1 : 0) + p.n_qb;
}

// lane l ^ M's value (M < 32: within each half of the wave; LDS crossbar, no memory access)
template <int M>
__device__ __forceinline__ float swz_xor(float v)
{
    static_assert(M > 0 && M < 32, "swizzle xor within 32 lanes");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
}

// max / sum over the RW consecutive lanes (RW a power of two) that hold this lane, in every
// lane of them.  Sixteen lanes: DPP within the row (rotations by 8 and 4, then the quad
// swaps); the max is the same in every lane, a sum may differ in its last bits between them.
template <int RW>
__device__ __forceinline__ float seg_max(float v)
{
    if constexpr (RW == 16) {
        v = dpp_max_step<0x128, 0xF>(v); // row_ror:8
        v = dpp_max_step<0x124, 0xF>(v); // row_ror:4
        v = dpp_max_step<0xB1, 0xF>(v);  // quad_perm [1,0,3,2]
        v = dpp_max_step<0x4E, 0xF>(v);  // quad_perm [2,3,0,1]
    } else {
        if constexpr (RW == 64)
            v = fmaxf(v, __shfl_xor(v, 32));
        if constexpr (RW >= 32)
            v = fmaxf(v, swz_xor<16>(v));
        if constexpr (RW >= 16)
            v = fmaxf(v, swz_xor<8>(v));
        v = fmaxf(v, swz_xor<4>(v));
        v = fmaxf(v, swz_xor<2>(v));
        v = fmaxf(v, swz_xor<1>(v));
    }
    return v;
}

template <int RW>
__device__ __forceinline__ float seg_sum(float v)
{
    if constexpr (RW == 16) {
        v = dpp_add_step<0x128, 0xF>(v);
        v = dpp_add_step<0x124, 0xF>(v);
        v = dpp_add_step<0xB1, 0xF>(v);
        v = dpp_add_step<0x4E, 0xF>(v);
    } else {
        if constexpr (RW == 64)
            v = v + __shfl_xor(v, 32);
        if constexpr (RW >= 32)
            v = v + swz_xor<16>(v);
        if constexpr (RW >= 16)
            v = v + swz_xor<8>(v);
        v = v + swz_xor<4>(v);
        v = v + swz_xor<2>(v);
        v = v + swz_xor<1>(v);
    }
    return v;
}


// The group energies' tree: level M adds lane l ^ M's partial sums (and takes the max of the
// largest |q|), for M = M0, M0/2, .., 1
template <int M, int CPL>
__device__ __forceinline__ void energy_tree(float (&sq)[CPL], float &am)
{
    if constexpr (M >= 1) {
#pragma unroll
        for (int s = 0; s < CPL; s++)
            sq[s] = sq[s] + swz_xor<M>(sq[s]);
        am = fmaxf(am, swz_xor<M>(am));
        energy_tree<M / 2, CPL>(sq, am);
    }
}

// sum over the 2M consecutive lanes holding this lane (xor butterfly M, M/2, .., 1)
template <int M>
__device__ __forceinline__ float bfly_sum(float v)
{
    if constexpr (M >= 1) {
        v = v + swz_xor<M>(v);
        v = bfly_sum<M / 2>(v);
    }
    return v;
}

// One wave per query head of the GQA group in every workgroup.  A record workgroup prepares
// one bucket of one unit: the stored-coordinate query (FWHT when keys are rotated), 16-channel
// group energies (fp32 stride-halving tree, the order the format fixes), the group's mask,
// and the head's query operands.  BF16 chunks of up to 64 positions each get the softmax
// state (m, l, o) of their positions per head, which the decode kernel folds into the unit's
// result: chunk 0, the sinks (in bucket 0's record workgroup, or in one of its own when there
// are many), and chunk c >= 1, the recent window's part of one 64-aligned block of positions
// (the chunks come first in the grid: the longest work).  REC: a grid of mostly record
// workgroups; with four heads it is compiled for eight waves per SIMD (at most 64 registers
// per lane), so the many short record workgroups (bucket-relative RoPE, large batches)
// overlap their latencies, while the chunk paths, which few of its workgroups take, keep some
// values in scratch.  A grid of mostly chunks takes the build without that bound.
template <int D, int G, int KF, bool REC>
__global__ __launch_bounds__(kWave * G, REC && G == 4 ? 8 : 2) void qprep_kernel(DecodeParams p)
{
    using C = Cfg<D, G, KF>;
    constexpr int KB = C::KB, KROWS = C::KROWS, PPW = C::PPW, NG = C::NG, NP = C::NP;
    constexpr int CPL = C::CPL, QW = C::QW;
    // a chunk's rows per wave (its workgroup's waves split the rows), and the value-row
    // registers: a wave's share of a chunk, or the few sinks of a record workgroup
    constexpr int RW = kWave / G;
    constexpr int NVR = RW > 2 * kSinksInRecord ? RW : 2 * kSinksInRecord;
    // A chunk lane holds the channels of one of the G parts of its key row (CPP channels, KQ
    // 16-byte words).  The scaled, masked queries sit in LDS with 4 words of padding after each
    // part (and 4 more per head), so the lanes of the G parts read them from different banks.
    constexpr int CPP = D / G, KQ = CPP / 8, SQS = D + 4 * G + 4;
    __shared__ float sq_[G * SQS];
    auto sqi = [](int g, int c) { return g * SQS + c + 4 * (c / CPP); };
    __shared__ float su_[G][D];     // the masked query before the softmax scale
    __shared__ float se[G][NP];
    __shared__ float sam[G][NP];
    __shared__ float cpo[G][G][D]; // a chunk's partial states: [row share][head]
    __shared__ float cpm[G][G], cpl[G][G];
    __shared__ uint32_t shalf[G][D]; // a head's fp16 query halves per channel (high | residual << 16)
    __shared__ int ssharp[G];

    const int lane = threadIdx.x % kWave;
    const int h = (int)uniform(threadIdx.x / kWave); // this wave's head (a chunk's row share)
    const int U = p.n_units;
    const bool sink_wg = p.n_sink > kSinksInRecord;
    const int nwin = U * (p.n_bch - 1), nsk = sink_wg ? U : 0;
    const int bi = (int)blockIdx.x;
    const bool wchunk = bi < nwin;                  // a window chunk's workgroup
    const bool chunk_only = bi < nwin + nsk;        // a chunk's workgroup (window or sinks)
    const int bid = wchunk ? bi : chunk_only ? bi - nwin : bi - nwin - nsk;
    const int unit = bid % U;
    const int grp = chunk_only ? 0 : bid / U;       // a record workgroup's bucket
    const int ch = wchunk ? 1 + bid / U : 0;        // BF16 chunk: 0 the sinks, c >= 1 the window's
    const bool state = chunk_only || (grp == 0 && !sink_wg); // computes chunk ch's softmax state
    const int b = unit / p.n_kv_heads;
    const int kvh = unit % p.n_kv_heads;
    const int n_q_heads = p.n_kv_heads * G;

    // this head's query as given: its raw words are loaded first (the first thing waited
    // for), converted after the row loads below have gone out
    uint32_t qw[CPL];
    {
        const size_t qoff = ((size_t)b * n_q_heads + (size_t)kvh * G + h) * D + (size_t)lane * CPL;
        if (p.q_bf16) {
            // (CPL = 2: both bf16 channels in one word, split when converted)
            const uint16_t *qb = static_cast<const uint16_t *>(p.q) + qoff;
            qw[0] = CPL == 2 ? *reinterpret_cast<const uint32_t *>(qb) : (uint32_t)qb[0];
            if constexpr (CPL == 2)
                qw[1] = 0u;
        } else {
            const uint32_t *qf = static_cast<const uint32_t *>(p.q) + qoff;
#pragma unroll
            for (int s = 0; s < CPL; s++)
                qw[s] = qf[s];
        }
    }

    // The chunk's BF16 rows: row j < nrows is position pos0 + j -- sink j (sink_k / sink_v), or
    // a window position in ring slot t mod W (Dual-QK sec. 3.3 / 4.1), the slots of a chunk
    // taken from one wrap point.  Window chunks are the window's part of the 64-aligned
    // position blocks, so none crosses a RoPE bucket edge (buckets are multiples of 128
    // positions).  The loads go out right after the query's (which are waited for first), so
    // their latency overlaps the query work.  Wave h takes rows h*RW .. h*RW + RW - 1: lane l
    // loads the whole key row h*RW + l % RW (the lanes of the G heads load the same rows), and
    // its CPL channels of each of the wave's value rows; registers of rows past nrows hold
    // zeros.
    const int ns_all = p.n_sink < p.len ? p.n_sink : p.len;
    const int wlo = p.q_end > ns_all ? p.q_end : ns_all; // first window position
    int pos0 = 0, nrows = 0;
    if (state) {
        if (ch == 0) {
            nrows = ns_all;
        } else {
            const int a0 = (wlo / kWave + ch - 1) * kWave; // the chunk's aligned block
            pos0 = wlo > a0 ? wlo : a0;
            nrows = (p.len < a0 + kWave ? p.len : a0 + kWave) - pos0;
        }
    }
    const uint16_t *kbase = ch == 0 ? p.sink_k : p.recent_k;
    const uint16_t *vbase = ch == 0 ? p.sink_v : p.recent_v;
    const int slot0 = ch == 0 ? 0 : pos0 % p.n_recent;
    auto row_off = [&](int j) -> size_t {
        const int jj = j < nrows ? j : nrows - 1;
        if (ch == 0)
            return ((size_t)unit * p.n_sink + (size_t)jj) * D;
        const int sl = slot0 + jj;
        return ((size_t)unit * p.n_recent + (size_t)(sl >= p.n_recent ? sl - p.n_recent : sl)) * D;
    };
    // A record workgroup's chunk (at most kSinksInRecord sinks) takes the few-rows path
    // instead: every lane loads its CPL channels of each sink row, key j into vr[j] and value
    // j into vr[kSinksInRecord + j]; each sink's logit is one wave-wide sum.
    const bool few = state && !chunk_only;
    uint4 kr[KQ];     // part lane / RW of key row h*RW + lane % RW (bf16; rows past nrows: zeros)
    uint32_t vr[NVR]; // value rows: this lane's CPL bf16 channels of row j (CPL = 1: low half)
    const int jrow = h * RW + lane % RW; // the row this lane scores
    if (few) {
#pragma unroll
        for (int j = 0; j < kSinksInRecord; j++) {
            if (j < nrows) {
                const size_t off = ((size_t)unit * p.n_sink + (size_t)j) * D + (size_t)lane * CPL;
                vr[j] = CPL == 2 ? *reinterpret_cast<const uint32_t *>(p.sink_k + off) : (uint32_t)p.sink_k[off];
                vr[kSinksInRecord + j] =
                    CPL == 2 ? *reinterpret_cast<const uint32_t *>(p.sink_v + off) : (uint32_t)p.sink_v[off];
            } else {
                vr[j] = vr[kSinksInRecord + j] = 0u;
            }
        }
    } else if (nrows > 0) {
        const uint4 *krow = reinterpret_cast<const uint4 *>(kbase + row_off(jrow)) + (lane / RW) * KQ;
#pragma unroll
        for (int c = 0; c < KQ; c++)
            kr[c] = jrow < nrows ? krow[c] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int jr = 0; jr < RW; jr++) {
            if (h * RW + jr < nrows) {
                const uint16_t *vrow = vbase + row_off(h * RW + jr) + (size_t)lane * CPL;
                vr[jr] = CPL == 2 ? *reinterpret_cast<const uint32_t *>(vrow) : (uint32_t)vrow[0];
            } else {
                vr[jr] = 0u;
            }
        }
    }

    // the bucket this workgroup prepares (a chunk's own; the sinks': 0) and, under
    // bucket-relative RoPE, the (cos, sin) of its anchor for this lane's channels
    const int bk = chunk_only ? (wchunk && p.rope_lw ? pos0 >> p.rope_lw : 0) : grp;
    float2 csr[CPL];
    if (p.rope_lw)
        anchor_cs<CPL>(csr, p.rope_cs + (size_t)bk * D, lane);

    float yq[CPL];
#pragma unroll
    for (int s = 0; s < CPL; s++)
        yq[s] = p.q_bf16 ? bf16_to_f32(s == 0 ? qw[0] & 0xFFFFu : qw[0] >> 16) : __uint_as_float(qw[s]);
    const float qscale = p.sm_log2e / (p.rotate ? (float)D : 1.0f);

    // Sharp query (Dual-QK sec. 1 and 3.2: query energy concentrated in a few channels): fewer
    // than five channels of the head with |q_c| at or above an eighth of its largest, in the
    // coordinates the query is given in (channel 0 left out when it is scored from its BF16
    // copy).  A unit with a sharp head gets a second, residual fp16 half per channel (about 22
    // bits per channel in all); one half keeps 11 bits relative to each channel, which the
    // logits of a few very large channels outgrow.
    if (!chunk_only) {
        float v[CPL], lm = 0.0f;
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            v[s] = (p.ch0 && lane * CPL + s == 0) ? 0.0f : fabsf(yq[s]);
            lm = fmaxf(lm, v[s]);
        }
        const float m1 = wave_max_dpp(lm);
        const float t = m1 * 0.125f;
        int big = 0;
#pragma unroll
        for (int s = 0; s < CPL; s++)
            big += __popcll(__ballot(v[s] >= t));
        if (lane == 0)
            ssharp[h] = m1 > 0.0f && big < 5 ? 1 : 0;
    }

    // The query of the bucket in stored coordinates (rotated back by the bucket's anchor
    // under bucket-relative RoPE, Dual-QK sec. 3.4 / C.4; then Walsh-Hadamard when keys are
    // rotated), its group energies (se) and largest |q| per group (sam; channel 0 left out
    // when it is scored from its BF16 copy), the mask, and this head's masked query (ym,
    // su_[h]) and scaled, masked query (sq_[h]).
    float ym[CPL];
    {
        float y[CPL];
#pragma unroll
        for (int s = 0; s < CPL; s++)
            y[s] = yq[s];
        if (p.rope_lw)
            anchor_apply<CPL>(y, csr, lane);
        if (p.rotate)
            fwht_wave<CPL>(y, lane);
        float sq[CPL], am = 0.0f;
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            ym[s] = y[s];
            sq[s] = y[s] * y[s];
            am = fmaxf(am, (p.ch0 && lane * CPL + s == 0) ? 0.0f : fabsf(y[s]));
        }
        // stride-halving tree over the 16 channels of a group: lanes of one group are
        // 16/CPL consecutive lanes; the xor butterfly reproduces the tree's sums.
        energy_tree<8 / CPL, CPL>(sq, am);
        float e = sq[0];
        if constexpr (CPL == 2)
            e = sq[0] + sq[1];
        if ((lane % (16 / CPL)) == 0) {
            se[h][lane / (16 / CPL)] = e;
            sam[h][lane / (16 / CPL)] = am;
        }
    }
    if (!chunk_only && grp == 0) {
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
    __syncthreads();

    // mask (every wave computes the same one): keep the `keep` highest group energies summed
    // over the heads in ascending head order, ties to the lower group.  Lane g < NP ranks
    // group g against the others' sums (read from their lanes).
    uint32_t mask = (1u << NP) - 1u;
    if (p.keep > 0 && p.keep < NP) {
        const int g = lane < NP ? lane : NP - 1;
        float eg = se[0][g];
#pragma unroll
        for (int hh = 1; hh < G; hh++)
            eg = eg + se[hh][g];
        int rank = 0;
#pragma unroll
        for (int o = 0; o < NP; o++) {
            const float eo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(eg), o));
            rank += (eo > eg || (eo == eg && o < g)) ? 1 : 0;
        }
        mask = (uint32_t)__ballot(lane < NP && rank < p.keep);
    }
    mask = uniform(mask);
#pragma unroll
    for (int s = 0; s < CPL; s++) {
        const int c = lane * CPL + s;
        const bool kept = (mask >> (c / 16)) & 1u;
        ym[s] = kept ? ym[s] : 0.0f;
        su_[h][c] = ym[s];
        sq_[sqi(h, c)] = ym[s] * qscale;
    }
    __syncthreads();

    // ---- the chunk's softmax state per head (the query of the chunk's bucket): log2 max m,
    // sum l and o = sum_t 2^(l_t - m) v_t over its positions, written by wave h for head h.
    // An empty chunk (no sinks) writes the empty state.  (Before the record: the chunk's rows
    // then leave the registers first.)
    if (state) {
        float M = -__builtin_inff(), L = 0.0f;
        float o[CPL];
#pragma unroll
        for (int s = 0; s < CPL; s++)
            o[s] = 0.0f;
        if (few && nrows > 0) {
            // (lane owns channels lane*CPL..: sink j's logit is a wave-wide sum; lane j keeps it)
            float qo[CPL];
#pragma unroll
            for (int s = 0; s < CPL; s++)
                qo[s] = sq_[sqi(h, lane * CPL + s)];
            float mine = -__builtin_inff();
#pragma unroll
            for (int j = 0; j < kSinksInRecord; j++) {
                if (j < nrows) {
                    float part = qo[0] * bf16_to_f32(vr[j] & 0xFFFFu);
                    if constexpr (CPL == 2)
                        part = fmaf(qo[1], bf16_to_f32(vr[j] >> 16), part);
                    const float tot = wave_sum_dpp(part);
                    mine = lane == j ? tot : mine;
                }
            }
            M = wave_max_dpp(mine);
            const float pw = lane < nrows ? __builtin_amdgcn_exp2f(mine - M) : 0.0f;
            L = wave_sum_dpp(pw);
#pragma unroll
            for (int j = 0; j < kSinksInRecord; j++) {
                if (j < nrows) {
                    const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), j));
                    const uint32_t v = vr[kSinksInRecord + j];
                    o[0] = fmaf(pj, bf16_to_f32(v & 0xFFFFu), o[0]);
                    if constexpr (CPL == 2)
                        o[1] = fmaf(pj, bf16_to_f32(v >> 16), o[1]);
                }
            }
        } else if (nrows > 0) {
            // Wave h's share of the rows for every head: the G lanes l % RW + k * RW hold the G
            // parts of row jrow; each scores its part against every head's masked, scaled query
            // (four partial sums, sum e taking channels 8i + 2e and 8i + 2e + 1: short dependency
            // chains), the parts are summed over those lanes (an xor butterfly: every lane of the
            // row gets the same sums), and lane l keeps head l / RW's.  Then the share's max and
            // sum per head over its RW lanes, and every lane sums its CPL channels of the share's
            // value rows for every head.  The shares' states meet in LDS; wave h merges head h's.
            const int hl = lane / RW; // the head this lane keeps (and the part it holds)
            float dg[G];
#pragma unroll
            for (int g = 0; g < G; g++) {
                float dp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int c = 0; c < KQ; c++) {
                    const uint32_t kk[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
                    const int c0 = hl * CPP + 8 * c;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        dp[e] = fmaf(sq_[sqi(g, c0 + 2 * e)], bf16_to_f32(kk[e] & 0xFFFFu), dp[e]);
                        dp[e] = fmaf(sq_[sqi(g, c0 + 2 * e + 1)], bf16_to_f32(kk[e] >> 16), dp[e]);
                    }
                }
                dg[g] = (dp[0] + dp[1]) + (dp[2] + dp[3]);
            }
#pragma unroll
            for (int o = RW; o < kWave; o <<= 1)
#pragma unroll
                for (int g = 0; g < G; g++)
                    dg[g] += __shfl_xor(dg[g], o);
            float dot = dg[0];
#pragma unroll
            for (int g = 1; g < G; g++)
                dot = hl == g ? dg[g] : dot;
            const bool valid = jrow < nrows;
            const float lw = valid ? dot : -__builtin_inff();
            const float mw = seg_max<RW>(lw); // -inf for a share without rows
            const float pw = valid ? __builtin_amdgcn_exp2f(lw - mw) : 0.0f;
            const float lsum = seg_sum<RW>(pw);
            float ow[G][CPL];
#pragma unroll
            for (int g = 0; g < G; g++)
#pragma unroll
                for (int s = 0; s < CPL; s++)
                    ow[g][s] = 0.0f;
#pragma unroll
            for (int jr = 0; jr < RW; jr++) {
                if (h * RW + jr < nrows) { // (a uniform test: the loop stays unrolled, vr in registers)
#pragma unroll
                    for (int g = 0; g < G; g++) {
                        const float pj =
                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), g * RW + jr));
                        ow[g][0] = fmaf(pj, bf16_to_f32(vr[jr] & 0xFFFFu), ow[g][0]);
                        if constexpr (CPL == 2)
                            ow[g][1] = fmaf(pj, bf16_to_f32(vr[jr] >> 16), ow[g][1]);
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < G; g++)
#pragma unroll
                for (int s = 0; s < CPL; s++)
                    cpo[h][g][lane * CPL + s] = ow[g][s];
            if (lane % RW == 0) {
                cpm[h][hl] = mw;
                cpl[h][hl] = lsum;
            }
            __syncthreads();
            // head h over the G shares (share 0 holds row 0: M is finite)
#pragma unroll
            for (int w = 0; w < G; w++)
                M = fmaxf(M, cpm[w][h]);
#pragma unroll
            for (int w = 0; w < G; w++) {
                const float f = __builtin_amdgcn_exp2f(cpm[w][h] - M); // (0 for a share without rows)
                L = fmaf(cpl[w][h], f, L);
#pragma unroll
                for (int s = 0; s < CPL; s++)
                    o[s] = fmaf(cpo[w][h][lane * CPL + s], f, o[s]);
            }
        }
        // the chunk's state, in the partial-state layout (m, l, two unused words, o[D])
        float *st = p.bstate + ((size_t)(unit * p.bch_max + ch) * G + h) * part_rec<D>();
        if (lane == 0) {
            st[0] = M;
            st[1] = L;
        }
#pragma unroll
        for (int s = 0; s < CPL; s++)
            st[4 + lane * CPL + s] = o[s];
    }

    if (chunk_only)
        return; // (a chunk's workgroup writes no record)

    // ---- the record of bucket bk
    bool sharp = false; // (ssharp is visible after the barriers)
#pragma unroll
    for (int hh = 0; hh < G; hh++)
        sharp = sharp || ssharp[hh] != 0;
    uint32_t *rec = p.qprep + ((size_t)unit * p.n_rb + bk) * C::QREC;
    float *recf = reinterpret_cast<float *>(rec);
    if (threadIdx.x == 0) {
        rec[C::OFF_MASK] = mask;
        rec[C::OFF_SHARP] = sharp ? 1u : 0u;
        if (p.mask_out)
            p.mask_out[(size_t)unit * p.n_rb + bk] = (uint8_t)mask;
    }
    if constexpr (KF == KVQ_K_LLOYD4) {
        // fp16 pairs of the query before the softmax scale (which goes into the fp32
        // accumulator unit), scaled so the largest kept |q| of the group lands in [2^12, 2^13);
        // byte j of key word r holds channels (8r + 2j, 8r + 2j + 1)
        float amax = 0.0f;
#pragma unroll
        for (int hh = 0; hh < G; hh++)
#pragma unroll
            for (int g = 0; g < NP; g++)
                amax = fmaxf(amax, (mask >> g & 1u) ? sam[hh][g] : 0.0f);
        int ex = 0;
        (void)frexpf(amax, &ex);
        const float g2 = amax > 0.0f ? ldexpf(1.0f, 13 - ex) : 1.0f;
        if (lane < KROWS * PPW) {
            const int r = lane / PPW, j = lane % PPW;
            const int ca = 8 * r + 2 * j;
            const float a = su_[h][ca] * g2, b2 = su_[h][ca + 1] * g2;
            const uint32_t hi = pack_f16x2(a, b2);
            rec[C::OFF_QP + (r * G + h) * QW + j] = hi;
            rec[C::OFF_QPL + (r * G + h) * QW + j] = sharp ? pack_f16x2(a - lo_f16(hi), b2 - hi_f16(hi)) : 0u;
        }
        if (lane == 0) {
            recf[C::OFF_QSC + h] = qscale / g2;
            recf[C::OFF_Q0 + h] = 0.0f;
        }
    } else {
        // fp16 query halves.  The decode kernel spreads a key word into registers whose two
        // halves hold the codes of channels (c, c + 32/KB/2) as subnormal integers
        // P(c) * code * 2^-24 (place factor P, see spread_asym), and multiplies them with
        // v_dot2_f32_f16 against halves q_c * g2 / P(c).  Every product is then
        // q~_c * g2 * code_c * 2^-24 with q~ the query rounded to fp16: each channel keeps 11
        // bits relative to its own magnitude, so one sharp query channel costs the others
        // nothing.  The halves hold the query before the softmax scale (which goes into the
        // fp32 accumulator unit), and g2 (a power of two) puts the head's largest kept |q| (the
        // largest of the kept groups' maxima) in [2^12, 2^13): a bf16 query is then carried
        // exactly.  Channel 0 (when protected) is scored from its BF16 copy: its half is 0.
        float am = 0.0f;
#pragma unroll
        for (int g = 0; g < NP; g++)
            am = fmaxf(am, (mask >> g & 1u) ? sam[h][g] : 0.0f);
        int ex = 0;
        (void)frexpf(am, &ex);
        const float g2 = am > 0.0f ? ldexpf(1.0f, 13 - ex) : 1.0f;
        // this lane's channels: the half of channel c (0 for the protected channel 0) and, for
        // a sharp query, the half of what it leaves (the residual, exact in fp32; g2 and the
        // place factors are powers of two); the zero-term sum of the query as the halves carry
        // it, in accumulator units g2 * 2^-24, over each 32-channel group (lanes of a group:
        // 32/CPL consecutive lanes)
        float si = 0.0f;
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            const int c = lane * CPL + s;
            const float x = (p.ch0 && c == 0) ? 0.0f : ym[s] * (g2 * asym_inv_place<KB>(c));
            const uint32_t hv = f32_to_f16(x);
            const uint32_t lv = sharp ? f32_to_f16(x - f16_to_f32(hv)) : 0u;
            si += (f16_to_f32(hv) + f16_to_f32(lv)) * (asym_place<KB>(c) * 0x1p-24f);
            shalf[h][c] = hv | (lv << 16);
        }
        // (the halves go to the lanes of the key words that hold their channels: within the wave)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // key word r, spread register k: halves hold channels asym_chan<KB>(r, k, 0 / 1)
        if (lane < KROWS * QW) {
            const int r = lane / QW, k = lane % QW;
            const uint32_t a0 = shalf[h][asym_chan<KB>(r, k, 0)], a1 = shalf[h][asym_chan<KB>(r, k, 1)];
            rec[C::OFF_QP + (r * G + h) * QW + k] = (a0 & 0xFFFFu) | (a1 << 16);
            rec[C::OFF_QPL + (r * G + h) * QW + k] = (a0 >> 16) | (a1 & 0xFFFF0000u);
        }
        si = bfly_sum<16 / CPL>(si);
        if (lane % (32 / CPL) == 0)
            recf[C::OFF_QZ + h * NG + lane / (32 / CPL)] = si;
        if (lane == 0) {
            recf[C::OFF_QSC + h] = qscale * (0x1p24f / g2);
            recf[C::OFF_Q0 + h] = (p.ch0 && (mask & 1u)) ? ym[0] * (g2 * 0x1p-24f) : 0.0f;
        }
    }
}

// ===================================================================== decode
template <int D, int G, int KF, int VF>
struct Smem {
    using C = Cfg<D, G, KF, VF>;
    uint32_t lut[KF == KVQ_K_LLOYD4 ? 256 : 1];      // Lloyd-Max code-pair table (fp16x2)
    uint32_t lutl[KF == KVQ_K_LLOYD4 ? 256 : 1];     // its residuals: centroid - fp16(centroid) (fp16x2)
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

// Asymmetric-key logits of this lane's TPL positions in accumulator units (g2 * 2^-24 per
// log2-logit unit, see the query prep):
//   lg = sum_g s_g * (q~ . code)_g + z_g * sum_{c in g} q~_c  (+ k0 * q0)
// ALL: every 16-channel row is kept (no pruning), so the row tests fold away.
// Per (group, head, position) one fp32 sum collects the dot2 products of the group's spread
// registers with the fp16 query halves (exact products, fp32 sums), then takes the group's
// scale and zero.  PREC (sharp queries): the residual halves go through the same spread
// registers too.  The query operands are uniform loads from the unit's record.
template <int D, int G, int KF, int VF, bool ALL, bool CH0, bool PREC>
__device__ __forceinline__ void score_asym(const KTile<D, G, KF, VF> &cur, const uint32_t *__restrict__ rec,
                                           uint32_t mask, float (&lg)[Cfg<D, G, KF>::TPL][G])
{
    using C = Cfg<D, G, KF>;
    constexpr int KB = C::KB, KROWS = C::KROWS, NG = C::NG, TPL = C::TPL, QW = C::QW;
    constexpr int RPG = KROWS / NG; // key rows per scale group
    const float *recf = reinterpret_cast<const float *>(rec);
#pragma unroll
    for (int g = 0; g < NG; g++) {
        if (!ALL && !(mask >> (2 * g) & 3u))
            continue;
        float a[G][TPL];
#pragma unroll
        for (int rr = 0; rr < RPG; rr++) {
            const int r = g * RPG + rr;
            if (!ALL && !(mask >> (r / C::RPP) & 1u)) {
                if (rr == 0) {
#pragma unroll
                    for (int h = 0; h < G; h++)
#pragma unroll
                        for (int i = 0; i < TPL; i++)
                            a[h][i] = 0.0f;
                }
                continue;
            }
#pragma unroll
            for (int i = 0; i < TPL; i++) {
                uint32_t sp[QW];
                spread_asym<KB>(i == 0 ? cur.kc[r].x : cur.kc[r].y, sp);
#pragma unroll
                for (int h = 0; h < G; h++) {
#pragma unroll
                    for (int k = 0; k < QW; k++)
                        a[h][i] = (rr == 0 && k == 0) ? dot2_first(sp[k], rec[C::OFF_QP + (r * G + h) * QW + k])
                                                      : dot2(sp[k], rec[C::OFF_QP + (r * G + h) * QW + k], a[h][i]);
                    if constexpr (PREC) {
#pragma unroll
                        for (int k = 0; k < QW; k++)
                            a[h][i] = dot2(sp[k], rec[C::OFF_QPL + (r * G + h) * QW + k], a[h][i]);
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float qz = recf[C::OFF_QZ + h * NG + g];
#pragma unroll
            for (int i = 0; i < TPL; i++) {
                const uint32_t szw = i == 0 ? cur.ksz[g].x : cur.ksz[g].y;
                lg[i][h] = fmaf(hi_f16(szw), qz, fmaf(lo_f16(szw), a[h][i], lg[i][h]));
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
// W / U members, one more for the first W mod U units.  Member k of n scores the k-th of n
// contiguous shares of the unit's first three quarters of tiles; the rest come from the
// unit's counter in the order the members ask, so a member that gets more issue slots takes
// more of them and the whole team ends together.  Teams of more than kStripe members work
// the same way on stripes of the unit (see the decode kernel).  In the deterministic mode
// the shares cover all the tiles.
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

// Combine the partial softmax states (m, l, o) of a unit's team, member k in slot u + k * U,
// with the states of its BF16 chunks: one global softmax over all positions (Dual-QK sec. 3.4),
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

// A batch of the states of two arrays taken as one sequence: records 0 .. n1 - 1 are those
// of r1 (ub1, ub1 + st1, ... bytes), the next ones those of r2 (ub2, ub2 + st2, ...); `total`
// states in all.  (The m / l lanes load from both arrays and keep the one that applies.)
template <int D, int G>
__device__ __forceinline__ void load_batch_two(CombineBatch<D, G> &b, rsrc_t r1, uint32_t ub1, uint32_t st1, int n1,
                                               rsrc_t r2, uint32_t ub2, uint32_t st2, int k0, int total, int lane)
{
    using CB = CombineBatch<D, G>;
    constexpr int CPL = CB::CPL, NB = CB::NB, PR = part_rec<D>();
    const int jm = lane % NB, hm = lane / NB;
    const int idx = k0 + jm;
    const bool mine = hm < G && idx < total, in1 = idx < n1;
    const uint32_t hb = (uint32_t)(mine ? hm : 0) * PR * 4u;
    const uint32_t p1 = ub1 + (uint32_t)(in1 ? idx : 0) * st1 + hb;
    const uint32_t p2 = ub2 + (uint32_t)(in1 ? 0 : idx - n1) * st2 + hb;
    const float m1 = load_shared(r1, p1), l1 = load_shared(r1, p1 + 4u);
    const float m2 = load_shared(r2, p2), l2 = load_shared(r2, p2 + 4u);
    b.m = mine ? (in1 ? m1 : m2) : -__builtin_inff();
    b.l = mine ? (in1 ? l1 : l2) : 0.0f;
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const int k = k0 + j; // (uniform)
        const bool f = k < n1;
        const rsrc_t r = f ? r1 : r2;
        const uint32_t rec = f ? ub1 + (uint32_t)k * st1 : ub2 + (uint32_t)(k - n1) * st2;
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int s = 0; s < CPL; s++)
                b.o[h][j][s] = k < total ? load_shared(r, rec + ((uint32_t)h * PR + 4u + lane + 64u * s) * 4u) : 0.0f;
    }
}

// Fold `count` states into the state (M, L, O), in order; load(batch, k0) loads the batch of
// states k0 .. k0 + NB - 1 (double-buffered: the next batch is in flight during a fold).
template <int D, int G, typename Load>
__device__ __forceinline__ void fold_run(Load &&load, int count, float (&M)[G], float (&L)[G], float (&O)[G][D / 64])
{
    using CB = CombineBatch<D, G>;
    constexpr int CPL = CB::CPL, NB = CB::NB;
    CB cur, nxt;
    load(cur, 0);
    for (int k0 = 0; k0 < count; k0 += NB) {
        if (k0 + NB < count)
            load(nxt, k0 + NB);
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

// Fold `count` partial states (slots first, first + step, ... in units of records, of an
// array of `slots` records at `base`) into the state (M, L, O).
template <int D, int G>
__device__ __forceinline__ void fold_states(const float *base, int slots, int first, int step, int count, int lane,
                                            float (&M)[G], float (&L)[G], float (&O)[G][D / 64])
{
    constexpr int PR = part_rec<D>();
    const uint32_t stride = (uint32_t)step * G * PR * 4u; // bytes between the states
    const rsrc_t r = make_rsrc(base, (uint32_t)slots * G * PR * 4u);
    const uint32_t ub = (uint32_t)first * G * PR * 4u;    // first state, head 0
    fold_run<D, G>([&](CombineBatch<D, G> &b, int k0) { load_batch<D, G>(b, r, ub, stride, k0, count, lane); },
                   count, M, L, O);
}

// The unit's team, last step: fold unit u's BF16 chunk states, then `count` states (stripe or
// member states), and write the normalised output out_u[h][D].  The two runs are folded as
// one sequence, so the chunk states and the first member states arrive in one batch.
template <int D, int G>
__device__ __forceinline__ void combine_unit(const DecodeParams &p, int u, int first, int step, int count, int lane,
                                             float *out_u)
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
    const rsrc_t rb = make_rsrc(p.bstate, (uint32_t)(p.n_units * p.bch_max) * G * PR * 4u);
    const uint32_t ubb = (uint32_t)(u * p.bch_max) * G * PR * 4u, sb = (uint32_t)G * PR * 4u;
    const rsrc_t rp = make_rsrc(p.part, (uint32_t)p.n_waves * G * PR * 4u);
    const uint32_t ubp = (uint32_t)first * G * PR * 4u, sp = (uint32_t)step * G * PR * 4u;
    const int nb = p.n_bch, total = nb + count;
    fold_run<D, G>([&](CombineBatch<D, G> &b, int k0) {
        load_batch_two<D, G>(b, rb, ubb, sb, nb, rp, ubp, sp, k0, total, lane);
    }, total, M, L, O);
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
    fold_states<D, G>(p.part, p.n_waves, first, step, count, lane, M, L, O);
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
        for (int e = lane; e < 256; e += kWave) {
            const float a = p.codebook[e & 15], b2 = p.codebook[e >> 4];
            const uint32_t hi = pack_f16x2(a, b2);
            sm.lut[e] = hi;
            sm.lutl[e] = pack_f16x2(a - lo_f16(hi), b2 - hi_f16(hi));
        }
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
    float acc_to_logit[G];
    int qbk = 0; // bucket whose scales acc_to_logit hold
    auto load_scales = [&](int bq) {
        const float *recf = reinterpret_cast<const float *>(rec + (size_t)bq * C::QREC);
#pragma unroll
        for (int h = 0; h < G; h++) {
            acc_to_logit[h] = recf[C::OFF_QSC + h];
        }
    };
    load_scales(0);

    // ---- running softmax state of the current unit
    float acc[G][8];
    float bacc[G][KQ ? 8 : 1]; // KQV: sketch-bit sums per channel
    float zacc[G][NGV];
    float lsum[G];
    // Softmax state per head: msub = m - vexp, the running maximum m in the weights' units,
    // so m = msub + vexp (no register of its own).  A weight's exponent is
    // x = l - msub = l - m + vexp; the maximum is raised when some x exceeds the wave-uniform
    // threshold xthr = kSlack + vexp, i.e. a logit exceeds m + kSlack.  xthr is -inf while the
    // state is empty (every head's at once: logits are masked by position, the same for all
    // heads), so the first tile with a finite logit sets m.
    float xthr = -__builtin_inff();
    // Value weights carry a power of two 2^vexp (wave-uniform): the fp16 products p * s
    // (p < 2^kSlack, s a value scale) must stay finite and normal whatever the values'
    // magnitude.  vexp starts at kVexpMax and is lowered (the state rescaled, as for a raised
    // maximum) whenever a scale with s * 2^vexp >= 2^13 arrives, so p * s * 2^vexp < 2^15;
    // sthr holds the fp16 bits of the largest scale allowed, in both halves.  The weights
    // are 2^(l - msub) with msub = m - vexp, and the wave's state is (m - vexp, l, o).
    float msub[G];
    int vexp = kVexpMax;
    uint32_t sthr = vexp_thr(kVexpMax);
    auto reset = [&]() {
#pragma unroll
        for (int h = 0; h < G; h++) {
            lsum[h] = 0.0f;
            msub[h] = -(float)kVexpMax;
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
            // the state's maximum in the weights' units (they carry 2^vexp)
            const float mst = xthr == -__builtin_inff() ? -__builtin_inff() : msub[h];
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
                const rsrc_t pr = make_rsrc(p.part, (uint32_t)p.n_waves * G * part_rec<D>() * 4u);
                const uint32_t rb = ((uint32_t)x * G + h) * part_rec<D>() * 4u;
                if (lane == 0)
                    store_shared2(pr, rb, mst, ls);
                store_shared4(pr, rb + (4u + 8u * lane) * 4u, o[0], o[1], o[2], o[3]);
                store_shared4(pr, rb + (8u + 8u * lane) * 4u, o[4], o[5], o[6], o[7]);
            }
            __syncthreads();
        }
        // Every wave stores its partial state (m, l, o) in the slot of its place; the unit's
        // result folds those of its team with the states of its BF16 chunks.  A unit served
        // by one wave combines at once.  Otherwise each member counts itself in once its
        // states are stored (all of the wave's memory operations complete); the member that
        // arrives last combines the states (in member order, so the result does not depend on
        // which member that is).  A striped team does it in two steps: the last member of
        // each stripe folds the stripe's states into its first member's slot and then counts
        // the stripe in; the last stripe folds the stripes' states.
        // Hand-over between compute units: the states are written and read with the
        // device-coherence cache policy (sc1) and the arrival atomic is issued only after the
        // stores have completed (s_waitcnt 0); the release / acquire fences keep the compiler
        // from moving memory accesses across the atomic.  That the completed sc1 stores are
        // visible to sc1 loads from any compute unit is a property of this device's caches
        // (no cache-wide write-back or invalidate is issued).
        float *out_u = p.out + ((size_t)b * n_q_heads + (size_t)kvh * G) * D;
        __builtin_amdgcn_s_waitcnt(0);
        if (whole) {
            combine_unit<D, G>(p, u, u, p.n_units, 1, lane, out_u);
        } else {
            uint32_t arrived = 0;
            if (S == 1) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                if (lane == 0)
                    arrived = __hip_atomic_fetch_add(p.tile_ctr + 2 * p.n_waves + u, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                if ((int)uniform(arrived) == team - 1)
                    combine_unit<D, G>(p, u, u, p.n_units, team, lane, out_u);
            } else {
                const int sfirst = u + m0 * p.n_units; // place of the stripe's first member
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                if (lane == 0)
                    arrived = __hip_atomic_fetch_add(p.tile_ctr + p.n_waves + sfirst, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                if ((int)uniform(arrived) == nst - 1) {
                    combine_stripe<D, G>(p, sfirst, p.n_units, nst, lane);
                    __builtin_amdgcn_s_waitcnt(0);
                    uint32_t done = 0;
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                    if (lane == 0)
                        done = __hip_atomic_fetch_add(p.tile_ctr + 2 * p.n_waves + u, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                    if ((int)uniform(done) == S - 1)
                        combine_unit<D, G>(p, u, u, B * p.n_units, S, lane, out_u);
                }
            }
        }
    };

    // this wave's tiles.  A stripe's first NS tiles are cut into contiguous shares, member k
    // of nst taking share k; the rest are drawn from the stripe's counter by whichever member
    // asks (tile ts0 + NS + draw), which evens out the members' unequal issue rates.  Only
    // the tail draws: a draw per tile costs read bandwidth (every tile's loads would wait on
    // an atomic's return).  The counter is asked one tile ahead of the answer's use (lane
    // 0's atomic; its return travels with the tile loads), so the next tile's loads can
    // still go out a whole tile before its scoring: key-side words and value words of the
    // current tile are in registers, and value word pair `it` is reloaded with the next
    // tile's right after its last use.  In the deterministic mode every tile is static.
    KTile<D, G, KF, VF> cur;
    VWord vcur[VIT];
    reset();
    const Slabs sl = unit_slabs<D, G, KF, VF>(p, u);
    uint32_t *const ctr = p.tile_ctr + (u + m0 * p.n_units);
    const bool dynamic = p.dynamic && nst > 1;
    const int NT = ts1 - ts0;                                        // the stripe's tiles
    // its static tiles: all of them in the deterministic mode or when there are no more than
    // members, else three quarters but at least one per member
    const int NS = sgpr(dynamic && NT > nst ? max((NT * 3) / 4, nst) : NT);
    const int r0 = sgpr(ts0 + (int)((long long)smem * NS / nst));    // this member's share
    const int r1 = sgpr(ts0 + (int)((long long)(smem + 1) * NS / nst));
    uint32_t ask = 0;
    int t_first = r0;
    if (r0 >= r1) {
        // no static tile (fewer static tiles than members): the first tile is drawn
        uint32_t a0 = 0;
        if (dynamic && lane == 0)
            a0 = draw_tile(ctr);
        t_first = dynamic ? ts0 + NS + (int)uniform(a0) : ts1;
    }
    // the tile after this one's needs a draw: ask now
    if (dynamic && lane == 0 && t_first < ts1 && (t_first + 1 >= r1))
        ask = draw_tile(ctr);
    // the tile loop, compiled for every-row-kept or not (ALL) and channel 0 apart or not
    // (CH0), so that neither costs a branch per tile
    auto tiles = [&](auto all_c, auto ch0_c, auto rope_c, auto prec_c) {
        constexpr bool ALL = decltype(all_c)::value;
        constexpr bool CH0 = decltype(ch0_c)::value;
        constexpr bool RP = decltype(rope_c)::value;   // per-bucket records (bucket-relative RoPE)
        constexpr bool PREC = decltype(prec_c)::value; // sharp query: residual query halves too
        // mask of the tile in `cur` (its bucket's; without RoPE the unit's)
        uint32_t mcur = mask;
        {
            const int t = t_first;
            const uint32_t off = t < ts1 ? 0u : kNoAccess;
            if (RP && t < ts1)
                mcur = rec[(size_t)(t >> tlw) * C::QREC + C::OFF_MASK];
            load_ktile<D, G, KF, VF, ALL, CH0>(cur, sl, ucap, lane, t * TILE, mcur, off);
#pragma unroll
            for (int it = 0; it < VIT; it++)
                vcur[it] = vload<V2>(sl.vc, vvo + off, ((uint32_t)(t * TILE / 2 + it * PPI) * WPP) * 4u);
        }
        for (int t = t_first; t < ts1;) {
            const int t0 = t * TILE;
            const int tl = t0 + lane * TPL;
            // the tile after this one: the next of the share, else a drawn one (or none)
            const int tn = t + 1 < r1 ? t + 1 : dynamic ? ts0 + NS + (int)uniform(ask) : ts1;
            const bool more = tn < ts1;
            if (dynamic && more && lane == 0 && tn + 1 >= r1)
                ask = draw_tile(ctr);
            // progress through the stripe: through the share in the static part (scaled to
            // it), the tile itself in the drawn part
            set_priority_for(t < r1 ? (int)((long long)(t - r0) * NS / (r1 - r0)) : t - ts0, NT);

            // ---- scores (accumulator units; log2 logit = lg * acc_to_logit[h]).  The query
            // operands are read through an address that depends on the tile number (the
            // added term is always 0: t >= 0), so they are reloaded per tile from the scalar
            // cache rather than hoisted out of the loop into more scalar registers than exist.
            const int bt = RP ? t >> tlw : 0;
            const uint32_t *__restrict__ rq = rec + ((uint32_t)t >> 31) + (size_t)bt * C::QREC;
            if (RP && bt != qbk) {
                // a tile of another bucket: its scales (the raise test is in log2 units)
                load_scales(bt);
                qbk = bt;
            }
            float lg[TPL][G];
#pragma unroll
            for (int i = 0; i < TPL; i++)
#pragma unroll
                for (int h = 0; h < G; h++)
                    lg[i][h] = 0.0f;
            if constexpr (KF != KVQ_K_LLOYD4) {
                score_asym<D, G, KF, VF, ALL, CH0, PREC>(cur, rq, mcur, lg);
            } else if constexpr (ALL && !PREC) {
                // Every row kept: a two-stage pipeline over the rows.  Row r + 1's table
                // lookups and query words go out after row r's first products, so their
                // latency hides behind the rest of row r.  The LDS reads and the uniform
                // loads share one wait counter, and a wait for the scalar loads covers every
                // outstanding read: loads issued before a row's first products would be waited
                // for there.  The scheduling barriers keep this order (the compiler would move
                // the uniform loads next to their use).
                uint32_t pr[2][TPL][4];
                auto lookup = [&](uint32_t (&o)[TPL][4], int r) {
#pragma unroll
                    for (int i = 0; i < TPL; i++) {
                        const uint32_t x = i == 0 ? cur.kc[r].x : cur.kc[r].y;
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            o[i][j] = sm.lut[(x >> (8 * j)) & 0xFFu];
                    }
                };
                static_assert(G * C::QW % 4 == 0, "a row's query words in uint4 loads");
                uint4 qb[2][G * C::QW / 4]; // a row's query words (uniform)
                auto loadq = [&](uint4 (&o)[G * C::QW / 4], int r) {
                    const uint4 *q4 = reinterpret_cast<const uint4 *>(rq + C::OFF_QP + r * G * C::QW);
#pragma unroll
                    for (int e = 0; e < G * C::QW / 4; e++)
                        o[e] = q4[e];
                };
                lookup(pr[0], 0);
                loadq(qb[0], 0);
#pragma unroll
                for (int r = 0; r < KROWS; r++) {
                    uint32_t(&cp)[TPL][4] = pr[r & 1];
                    const uint4(&qc)[G * C::QW / 4] = qb[r & 1];
                    auto qword = [&](int h, int j) {
                        const uint4 v = qc[(h * C::QW + j) / 4];
                        const int e = (h * C::QW + j) % 4;
                        return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
                    };
#pragma unroll
                    for (int i = 0; i < TPL; i++)
                        lg[i][0] = dot2(cp[i][0], qword(0, 0), lg[i][0]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (r + 1 < KROWS) {
                        lookup(pr[(r + 1) & 1], r + 1);
                        loadq(qb[(r + 1) & 1], r + 1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int h = 0; h < G; h++)
#pragma unroll
                        for (int j = (h == 0 ? 1 : 0); j < 4; j++) {
#pragma unroll
                            for (int i = 0; i < TPL; i++)
                                lg[i][h] = dot2(cp[i][j], qword(h, j), lg[i][h]);
                        }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < TPL; i++) {
                    const float rho = f16_to_f32(i == 0 ? (cur.kx & 0xFFFFu) : (cur.kx >> 16));
#pragma unroll
                    for (int h = 0; h < G; h++)
                        lg[i][h] *= rho;
                }
            } else {
#pragma unroll
                for (int r = 0; r < KROWS; r++) {
                    if (!ALL && !(mcur >> (r / C::RPP) & 1u))
                        continue;
                    // (a sharp query also takes the centroids' fp16 residuals: the products
                    // hi.hi + hi.lo + lo.hi carry about 22 bits on either side)
                    uint32_t pr[TPL][4], prl[TPL][PREC ? 4 : 1];
#pragma unroll
                    for (int i = 0; i < TPL; i++) {
                        const uint32_t x = i == 0 ? cur.kc[r].x : cur.kc[r].y;
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            pr[i][j] = sm.lut[(x >> (8 * j)) & 0xFFu];
                            if constexpr (PREC)
                                prl[i][j] = sm.lutl[(x >> (8 * j)) & 0xFFu];
                        }
                    }
#pragma unroll
                    for (int h = 0; h < G; h++)
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            const uint32_t qv = rq[C::OFF_QP + (r * G + h) * C::QW + j];
#pragma unroll
                            for (int i = 0; i < TPL; i++)
                                lg[i][h] = dot2(pr[i][j], qv, lg[i][h]);
                            if constexpr (PREC) {
                                const uint32_t ql = rq[C::OFF_QPL + (r * G + h) * C::QW + j];
#pragma unroll
                                for (int i = 0; i < TPL; i++)
                                    lg[i][h] = dot2(prl[i][j], qv, dot2(pr[i][j], ql, lg[i][h]));
                            }
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

            // ---- value scales of this lane's positions as fp16 pairs (s0, s1), and the zero
            // points (z0, z1) (KQV: residual norms); is any scale too large for vexp?
            uint32_t spair[NGV], zpair[NGV];
#pragma unroll
            for (int gg = 0; gg < NGV; gg++) {
                spair[gg] = __builtin_amdgcn_perm(vsw[1][gg], vsw[0][gg], 0x05040100u);
                zpair[gg] = __builtin_amdgcn_perm(vsw[1][gg], vsw[0][gg], 0x07060302u);
            }
            uint32_t smx = spair[0];
#pragma unroll
            for (int gg = 1; gg < NGV; gg++)
                smx = max_u16x2(smx, spair[gg]);
            if constexpr (KQ)
                smx = max_u16x2(smx, zpair[0]);
            const uint64_t s_above = __ballot(max_u16x2(smx, sthr) != sthr);

            // ---- online softmax (log2 units), per head.  The running maximum m is raised
            // (wave-wide DPP max, rescale of that head's state) only when a logit exceeds
            // m + kSlack; otherwise weights 2^(l - m) may reach 2^kSlack, and the raise is
            // rare after the first tile.  The weights' exponents x = l - msub are computed
            // first and their lane maximum is tested against xthr = kSlack + vexp (one compare
            // for all heads and positions); a rounding miss is harmless.  A value scale beyond
            // sthr lowers vexp in the same branch (every head's state rescaled).  One branch
            // per tile covers all heads: one per head splits the tile's code into blocks the
            // compiler cannot schedule across, which costs far more than the raises
            // themselves (about one per two tiles over all heads).
            float xw[TPL][G];
            float xmx = -__builtin_inff();
#pragma unroll
            for (int h = 0; h < G; h++)
#pragma unroll
                for (int i = 0; i < TPL; i++) {
                    xw[i][h] = fmaf(lg[i][h], acc_to_logit[h], -msub[h]);
                    xmx = fmaxf(xmx, xw[i][h]);
                }
            if (s_above | __ballot(xmx > xthr)) {
                int enew = vexp;
                if (s_above) {
                    // the wave's largest scale: 2^(e-15) <= s < 2^(e-14) for exponent field e,
                    // so vexp = 27 - e keeps s * 2^vexp below 2^13; kVexpRoom binades lower
                    // (not below -3, which admits every finite scale) leaves room for larger
                    // scales to come
                    const uint32_t lm = (smx & 0xFFFFu) > (smx >> 16) ? (smx & 0xFFFFu) : (smx >> 16);
                    const int e = (int)wave_max_dpp((float)lm) >> 10;
                    enew = min(vexp, max(-3, 27 - kVexpRoom - e));
                }
                const float fe = ldexpf(1.0f, enew - vexp);
                bool filled = xthr != -__builtin_inff();
#pragma unroll
                for (int h = 0; h < G; h++) {
                    float xh = xw[0][h];
#pragma unroll
                    for (int i = 1; i < TPL; i++)
                        xh = fmaxf(xh, xw[i][h]);
                    const bool above = __ballot(xh > xthr) != 0;
                    if (!above && enew == vexp)
                        continue;
                    const float mold = xthr == -__builtin_inff() ? -__builtin_inff() : msub[h] + (float)vexp;
                    float mnew = mold;
                    if (above) {
                        float mt = lg[0][h];
#pragma unroll
                        for (int i = 1; i < TPL; i++)
                            mt = fmaxf(mt, lg[i][h]);
                        mnew = fmaxf(mold, wave_max_dpp(mt * acc_to_logit[h]) + kRaiseRoom);
                    }
                    filled = filled || mnew != -__builtin_inff();
                    // (a state still empty, m = -inf, is all zeros: any finite factor keeps it)
                    const float alpha = mold == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mold - mnew) * fe;
                    // (a maximum still at -inf means every logit so far, this tile's included,
                    // is -inf: subtract -vexp instead so the weights come out 0, not NaN)
                    msub[h] = (mnew == -__builtin_inff() ? 0.0f : mnew) - (float)enew;
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
#pragma unroll
                    for (int i = 0; i < TPL; i++)
                        xw[i][h] = fmaf(lg[i][h], acc_to_logit[h], -msub[h]);
                }
                vexp = enew;
                sthr = vexp_thr(enew);
                xthr = filled ? kSlack + (float)enew : -__builtin_inff();
            }
            float pw[TPL][G];
#pragma unroll
            for (int h = 0; h < G; h++)
#pragma unroll
                for (int i = 0; i < TPL; i++)
                    pw[i][h] = __builtin_amdgcn_exp2f(xw[i][h]);
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
                const uint32_t sp = spair[gg], zp = zpair[gg];
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
    // by bucket; a sharp query takes the pruned-rows variant with the residual halves)
    constexpr bool ASYM = KF != KVQ_K_LLOYD4;
    const bool sharp = rec[C::OFF_SHARP] != 0u;
    const BoolC<true> T_;
    const BoolC<false> F_;
    if (p.rope_lw) {
        if (ASYM && p.ch0)
            sharp ? tiles(F_, BoolC<ASYM>(), T_, T_) : tiles(F_, BoolC<ASYM>(), T_, F_);
        else
            sharp ? tiles(F_, F_, T_, T_) : tiles(F_, F_, T_, F_);
    } else if (mask == (1u << NP) - 1u && !sharp) {
        if (ASYM && p.ch0)
            tiles(T_, BoolC<ASYM>(), F_, F_);
        else
            tiles(T_, F_, F_, F_);
    } else {
        if (ASYM && p.ch0)
            sharp ? tiles(F_, BoolC<ASYM>(), F_, T_) : tiles(F_, BoolC<ASYM>(), F_, F_);
        else
            sharp ? tiles(F_, F_, F_, T_) : tiles(F_, F_, F_, F_);
    }
    flush();
}

// ===================================================================== launchers
template <int D, int G, int KF, int VF>
hipError_t launch_one(int units, const DecodeParams &p, hipEvent_t const ev[2], hipStream_t s)
{
    // window chunks, the sinks' chunk (many sinks), then the record groups
    const unsigned qgrid = (unsigned)(qprep_groups(p) * units);
    const int chunk_wgs = (p.n_bch - 1 + (p.n_sink > kSinksInRecord ? 1 : 0)) * units;
    if ((int)qgrid - chunk_wgs >= 4 * chunk_wgs)
        hipLaunchKernelGGL((qprep_kernel<D, G, KF, true>), dim3(qgrid), dim3(kWave * G), 0, s, p);
    else
        hipLaunchKernelGGL((qprep_kernel<D, G, KF, false>), dim3(qgrid), dim3(kWave * G), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const uint32_t *qrec = static_cast<const uint32_t *>(p.qprep);
    if (ev[0] && ev[1]) {
        // measurement: the events are taken by the dispatch itself, at the start and the end
        // of the kernel's execution
        void *args[] = {const_cast<DecodeParams *>(&p), &qrec};
        return hipExtLaunchKernel(reinterpret_cast<const void *>(&decode_kernel<D, G, KF, VF>),
                                  dim3((unsigned)p.n_waves), dim3(kWave), args, 0, s, ev[0], ev[1], 0);
    }
    hipLaunchKernelGGL((decode_kernel<D, G, KF, VF>), dim3((unsigned)p.n_waves), dim3(kWave), 0, s, p, qrec);
    return hipGetLastError();
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
