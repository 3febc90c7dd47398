// kvq_append.hip -- quantize-and-pack of new key/value tokens into the low-bit cache.
//
// One wave encodes one (unit, position): 64 lanes hold head_dim/64 channels each.  The
// arithmetic is the format's fixed fp32 sequence, so the packed bytes are reproducible:
//   keys, asymmetric INT-b (Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV
//   Caches, sec. 3.3): per 32-channel group min/max (channel 0 left out when protected,
//   sec. C.3), fp16 scale = (max-min)/(2^b-1) and fp16 zero = min, codes against the
//   rounded parameters;
//   keys, Lloyd-Max (TurboQuant on Quantized Models, topic list; Statistical Inference ...
//   Inspired by TurboQuant, scheme KQV): optional Walsh-Hadamard rotation as a butterfly
//   across lanes, norm from the stride-halving tree of squares (an xor butterfly gives
//   the same sums bit for bit because fp32 addition commutes), fp16 norm, codes by
//   threshold count;
//   values: asymmetric INT4 per 32-channel group, or per-token asymmetric INT2 whose range
//   is clipped to [c*min, c*max] (Dual-QK sec. B.2: per-token INT2 values, clipping ratio);
//   positions below n_sink: BF16 keys and values (TurboQuant on Quantized Models, abstract);
//   with a recent window of W positions (Dual-QK sec. 3.3 / 4.1; past-only quantization),
//   new positions go to ring slot t mod W in BF16 and are quantised from that copy when they
//   leave the window (a first launch with `evict` set does those of earlier appends).
//   with bucket-relative RoPE (Dual-QK sec. 3.4 / C.4), keys are first rotated back by the
//   anchor of their position's bucket, before the Walsh-Hadamard rotation.
// Work per appended token is O(head_dim) and touches only that token's slots
// (TurboQuant on Quantized Models, abstract: incremental cache).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

#pragma clang fp contract(off)

template <int CPL>
__device__ __forceinline__ void load_row(const void *base, size_t off, int in_bf16, float (&x)[CPL])
{
    if (in_bf16) {
        const uint16_t *p = static_cast<const uint16_t *>(base) + off;
        if constexpr (CPL == 2) {
            uint32_t w = *reinterpret_cast<const uint32_t *>(p);
            x[0] = bf16_to_f32(w & 0xFFFFu);
            x[1] = bf16_to_f32(w >> 16);
        } else {
            x[0] = bf16_to_f32(*p);
        }
    } else {
        const float *p = static_cast<const float *>(base) + off;
        if constexpr (CPL == 2) {
            float2 w = *reinterpret_cast<const float2 *>(p);
            x[0] = w.x;
            x[1] = w.y;
        } else {
            x[0] = *p;
        }
    }
}

// Unnormalised Walsh-Hadamard transform of the wave's head_dim values; lane l holds
// channels CPL*l .. CPL*l+CPL-1.  Stage h combines channel j with j+h as (a+b, a-b).
template <int CPL>
__device__ __forceinline__ void fwht(float (&y)[CPL], int lane)
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

// Asymmetric b-bit quantization of this lane's channels within 32-channel groups spread
// over LPG = 32/CPL lanes.  skip0: exclude channel 0 (lane 0, slot 0) from min/max and
// code it as 0.  Returns codes and the group's packed fp16 (scale | zero << 16).
template <int CPL>
__device__ __forceinline__ uint32_t asym_quant(const float (&x)[CPL], int bits, bool skip0,
                                               int lane, uint32_t (&code)[CPL])
{
    constexpr int LPG = 32 / CPL;
    const float qmax = (float)((1 << bits) - 1);
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int s = 0; s < CPL; s++) {
        const bool excluded = skip0 && lane == 0 && s == 0;
        if (!excluded) {
            mn = fminf(mn, x[s]);
            mx = fmaxf(mx, x[s]);
        }
    }
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
    }
    // a zero minimum or range is stored as +0 whatever the scan order of -0 / +0
    mn = mn + 0.0f;
    const float range = (mx - mn) + 0.0f;
    const float scale32 = range / qmax;
    const uint32_t sh = f32_to_f16(scale32);
    const uint32_t zh = f32_to_f16(mn);
    const float sf = f16_to_f32(sh);
    const float zf = f16_to_f32(zh);
    const float inv = sf > 0.0f ? 1.0f / sf : 0.0f;
#pragma unroll
    for (int s = 0; s < CPL; s++) {
        const float diff = x[s] - zf;
        const float u = diff * inv;
        float r = __builtin_rintf(u);
        r = fminf(fmaxf(r, 0.0f), qmax);
        code[s] = (skip0 && lane == 0 && s == 0) ? 0u : (uint32_t)r;
    }
    return sh | (zh << 16);
}

// OR-combine the b-bit codes of `lanes` consecutive lanes into one word (lowest lane in
// the low bits); the combined value is valid in every lane of the run.
template <int CPL>
__device__ __forceinline__ uint32_t pack_run(const uint32_t (&code)[CPL], int bits, int lanes, int lane)
{
    uint32_t frag = 0;
#pragma unroll
    for (int s = 0; s < CPL; s++)
        frag |= code[s] << (bits * s);
    frag <<= (lane % lanes) * bits * CPL;
    for (int m = 1; m < lanes; m <<= 1)
        frag |= __shfl_xor(frag, m);
    return frag;
}

template <int D>
__global__ __launch_bounds__(kBlock) void append_kernel(AppendParams p)
{
    constexpr int CPL = D / 64;
    constexpr int NG = D / 32;
    const int lane = threadIdx.x & 63;
    const long long wave = (long long)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (wave >= (long long)p.units * p.n_new)
        return;
    const int u = (int)(wave / p.n_new);
    const int i = (int)(wave % p.n_new);
    const size_t cap = (size_t)p.cap;
    const size_t W = (size_t)p.n_recent;

    float k[CPL], v[CPL]; // the key in stored coordinates, the value
    int t;
    if (p.evict) {
        // position t leaves the recent window: quantise its BF16 copy from the ring
        t = p.e0 + i;
        const size_t ro = ((size_t)u * W + (size_t)t % W) * D + (size_t)lane * CPL;
        load_row<CPL>(p.recent_k, ro, 1, k);
        load_row<CPL>(p.recent_v, ro, 1, v);
    } else {
        t = p.len + i;
        const size_t in_off = ((size_t)u * (size_t)p.n_new + (size_t)i) * D + (size_t)lane * CPL;
        load_row<CPL>(p.k_new, in_off, p.in_bf16, k);
        load_row<CPL>(p.v_new, in_off, p.in_bf16, v);
        if (p.rope_lw)
            anchor_rotate<CPL>(k, p.rope_cs + (size_t)(t >> p.rope_lw) * D, lane);
        if (p.rotate)
            fwht<CPL>(k, lane);

        if (t < p.n_sink) {
            const size_t so = ((size_t)u * (size_t)p.n_sink + (size_t)t) * D + (size_t)lane * CPL;
#pragma unroll
            for (int s = 0; s < CPL; s++) {
                p.sink_k[so + s] = (uint16_t)f32_to_bf16(k[s]);
                p.sink_v[so + s] = (uint16_t)f32_to_bf16(v[s]);
            }
            return;
        }
        if (W > 0) {
            if (t >= p.q_end) {
                // still among the W most recent positions: into its ring slot, in BF16
                const size_t ro = ((size_t)u * W + (size_t)t % W) * D + (size_t)lane * CPL;
#pragma unroll
                for (int s = 0; s < CPL; s++) {
                    p.recent_k[ro + s] = (uint16_t)f32_to_bf16(k[s]);
                    p.recent_v[ro + s] = (uint16_t)f32_to_bf16(v[s]);
                }
                return;
            }
            // already W behind the new end: quantised from the BF16 copy it would have had
#pragma unroll
            for (int s = 0; s < CPL; s++) {
                k[s] = bf16_to_f32(f32_to_bf16(k[s]));
                v[s] = bf16_to_f32(f32_to_bf16(v[s]));
            }
        }
    }

    // ---- keys
    uint32_t code[CPL];
    int kbits;
    if (p.kfmt == KVQ_K_LLOYD4) {
        kbits = 4;
        float sq[CPL];
#pragma unroll
        for (int s = 0; s < CPL; s++)
            sq[s] = k[s] * k[s];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
            for (int s = 0; s < CPL; s++)
                sq[s] = sq[s] + __shfl_xor(sq[s], m);
        }
        float s2 = sq[0];
        if constexpr (CPL == 2)
            s2 = sq[0] + sq[1];
        const float rho32 = __builtin_sqrtf(s2 / (float)D);
        const uint32_t rh = f32_to_f16(rho32);
        const float rf = f16_to_f32(rh);
        const float inv = rf > 0.0f ? 1.0f / rf : 0.0f;
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            const float z = k[s] * inv;
            uint32_t c = 0;
#pragma unroll
            for (int j = 0; j < 15; j++)
                c += (z > p.thresholds[j]) ? 1u : 0u;
            code[s] = c;
        }
        if (lane == 0)
            p.k_norm[(size_t)u * cap + (size_t)t] = (uint16_t)rh;
    } else {
        kbits = (p.kfmt == KVQ_K_ASYM2) ? 2 : 4;
        const int g = lane * CPL / 32;
        const uint32_t sz = asym_quant<CPL>(k, kbits, p.ch0 && g == 0, lane, code);
        if ((lane % (32 / CPL)) == 0)
            p.k_sz[((size_t)u * NG + (size_t)g) * cap + (size_t)t] = sz;
        if (p.ch0 && lane == 0)
            p.k_ch0[(size_t)u * cap + (size_t)t] = (uint16_t)f32_to_bf16(k[0]);
    }
    {
        const int lanes = 32 / (kbits * CPL); // lanes contributing to one 32-bit row word
        const uint32_t word = pack_run<CPL>(code, kbits, lanes, lane);
        const int rows = D * kbits / 32;
        if ((lane % lanes) == 0)
            p.k_codes[((size_t)u * (size_t)rows + (size_t)(lane / lanes)) * cap + (size_t)t] = word;
    }

    // ---- values, KQV (Statistical Inference ... Inspired by TurboQuant, scheme KQV; TurboQuant
    // on Quantized Models, abstract: SRHT-QJL): y = FWHT(v), 3-bit Lloyd-Max codes of y / rho
    // (rho = RMS of y, fp16, as for keys), residual r = y - rho cent[code], sketch bits = signs
    // of FWHT(D r), residual norm in fp16; nibble = code | bit << 3 in the INT4 pair layout
    if (p.vfmt == KVQ_V_KQV) {
        float y[CPL], sq[CPL], r[CPL], w[CPL];
#pragma unroll
        for (int s = 0; s < CPL; s++)
            y[s] = v[s];
        fwht<CPL>(y, lane);
#pragma unroll
        for (int s = 0; s < CPL; s++)
            sq[s] = y[s] * y[s];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
            for (int s = 0; s < CPL; s++)
                sq[s] = sq[s] + __shfl_xor(sq[s], m);
        }
        float s2 = sq[0];
        if constexpr (CPL == 2)
            s2 = sq[0] + sq[1];
        const uint32_t rh = f32_to_f16(__builtin_sqrtf(s2 / (float)D));
        const float rf = f16_to_f32(rh);
        const float inv = rf > 0.0f ? 1.0f / rf : 0.0f;
        uint32_t vc[CPL];
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            const float z = y[s] * inv;
            uint32_t c = 0;
#pragma unroll
            for (int j = 0; j < 7; j++)
                c += (z > p.v_thresholds[j]) ? 1u : 0u;
            vc[s] = c;
            const float yh = rf * p.v_codebook[c];
            r[s] = y[s] - yh;
            const int ch = lane * CPL + s;
            w[s] = ((p.v_qjl[ch / 32] >> (ch % 32)) & 1u) ? -r[s] : r[s];
            sq[s] = r[s] * r[s];
        }
        fwht<CPL>(w, lane);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
            for (int s = 0; s < CPL; s++)
                sq[s] = sq[s] + __shfl_xor(sq[s], m);
        }
        float g2 = sq[0];
        if constexpr (CPL == 2)
            g2 = sq[0] + sq[1];
        const uint32_t gh = f32_to_f16(__builtin_sqrtf(g2));
#pragma unroll
        for (int s = 0; s < CPL; s++)
            vc[s] |= (w[s] < 0.0f ? 1u : 0u) << 3;
        if (lane == 0)
            p.v_sz[(size_t)u * cap + (size_t)t] = rh | (gh << 16);
        const int lanes = 16 / (4 * CPL); // lanes forming one 16-bit half (4 channels)
        const uint32_t half = pack_run<CPL>(vc, 4, lanes, lane);
        if ((lane % lanes) == 0) {
            const size_t word = ((size_t)u * (cap / 2) + (size_t)(t >> 1)) * (D / 4) + (size_t)(lane / lanes);
            reinterpret_cast<uint16_t *>(p.v_codes)[word * 2 + (size_t)(t & 1)] = (uint16_t)half;
        }
        return;
    }

    // ---- values, per-token INT2: range [c*min, c*max] over the whole token, codes against
    // the fp16 scale and zero, 8 channels per 16-bit half of a token-pair word
    if (p.vfmt == KVQ_V_ASYM2_TOKEN) {
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int s = 1; s < CPL; s++) {
            mn = fminf(mn, v[s]);
            mx = fmaxf(mx, v[s]);
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            mn = fminf(mn, __shfl_xor(mn, m));
            mx = fmaxf(mx, __shfl_xor(mx, m));
        }
        mn = p.vclip * mn + 0.0f;
        mx = p.vclip * mx;
        const float range = (mx - mn) + 0.0f;
        const float scale32 = range / 3.0f;
        const uint32_t sh = f32_to_f16(scale32);
        const uint32_t zh = f32_to_f16(mn);
        const float sf = f16_to_f32(sh);
        const float zf = f16_to_f32(zh);
        const float inv = sf > 0.0f ? 1.0f / sf : 0.0f;
        uint32_t vc[CPL];
#pragma unroll
        for (int s = 0; s < CPL; s++) {
            const float diff = v[s] - zf;
            const float uu = diff * inv;
            const float r = fminf(fmaxf(__builtin_rintf(uu), 0.0f), 3.0f);
            vc[s] = (uint32_t)r;
        }
        if (lane == 0)
            p.v_sz[(size_t)u * cap + (size_t)t] = sh | (zh << 16);
        const int lanes = 16 / (2 * CPL); // lanes forming one 16-bit half (8 channels)
        const uint32_t half = pack_run<CPL>(vc, 2, lanes, lane);
        if ((lane % lanes) == 0) {
            const size_t word = ((size_t)u * (cap / 2) + (size_t)(t >> 1)) * (D / 8) + (size_t)(lane / lanes);
            reinterpret_cast<uint16_t *>(p.v_codes)[word * 2 + (size_t)(t & 1)] = (uint16_t)half;
        }
        return;
    }

    // ---- values: asymmetric INT4, token-pair interleaved words
    {
        uint32_t vc[CPL];
        const int g = lane * CPL / 32;
        const uint32_t sz = asym_quant<CPL>(v, 4, false, lane, vc);
        if ((lane % (32 / CPL)) == 0)
            p.v_sz[((size_t)u * NG + (size_t)g) * cap + (size_t)t] = sz;
        const int lanes = 16 / (4 * CPL); // lanes forming one 16-bit half (4 channels)
        const uint32_t half = pack_run<CPL>(vc, 4, lanes, lane);
        if ((lane % lanes) == 0) {
            const size_t word = ((size_t)u * (cap / 2) + (size_t)(t >> 1)) * (D / 4) + (size_t)(lane / lanes);
            reinterpret_cast<uint16_t *>(p.v_codes)[word * 2 + (size_t)(t & 1)] = (uint16_t)half;
        }
    }
}

} // namespace

hipError_t launch_append(int head_dim, const AppendParams &p, hipStream_t s)
{
    const long long waves = (long long)p.units * p.n_new;
    const long long blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7FFFFFFFLL)
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks), block(kBlock);
    if (head_dim == 128)
        hipLaunchKernelGGL(append_kernel<128>, grid, block, 0, s, p);
    else
        hipLaunchKernelGGL(append_kernel<64>, grid, block, 0, s, p);
    return hipGetLastError();
}

} // namespace kvq
