// kvq_internal.h -- launcher interface between the C ABI (kvq_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;

// Decode tile: positions scored by one wave per pass (64 lanes x 2 positions).
constexpr int kTile = 128;
// Upper bound on decode waves per call when units share waves (one wave per resident slot).
constexpr int kMaxWaves = 16384;
// Cache capacity granule (public contract: capacity is a multiple of 256 positions).
constexpr int kCapacityQuantum = 256;
constexpr int kMaxSink = 64;
// Largest recent BF16 window (positions per sequence).
constexpr int kMaxRecent = 1024;
// Largest capacity (positions per sequence): keeps every per-unit slab under 1 GiB.
constexpr int kMaxCapacity = 1 << 24;

struct AppendParams {
    uint32_t *k_codes, *k_sz, *v_codes, *v_sz;
    uint16_t *k_norm, *k_ch0, *sink_k, *sink_v, *recent_k, *recent_v;
    const float *thresholds;
    const void *k_new, *v_new;
    int units, n_new, cap, len, n_sink, kfmt, rotate, ch0, vfmt, in_bf16;
    float vclip;  // per-token INT2 values: clipping ratio
    int n_recent; // recent BF16 window W (0: none)
    int q_end;    // positions below q_end (and >= n_sink) end up quantised by this append
    int evict;    // 1: quantise ring positions [len - ..., ) leaving the window (see the kernel)
    int e0;       // evict: first position to quantise; n_new positions from there
    const float *rope_cs; // bucket-relative RoPE: (cos, sin) of each bucket's anchor [bucket][D/2][2]
    int rope_lw;          // log2 of the bucket width, 0: off
    const float *v_codebook, *v_thresholds; // KQV values: 8 centroids, 7 thresholds
    const uint32_t *v_qjl;                  // KQV values: the sketch's sign diagonal (bit set: -1)
};

struct DecodeParams {
    const uint32_t *k_codes, *k_sz, *v_codes, *v_sz;
    const uint16_t *k_norm, *k_ch0, *sink_k, *sink_v, *recent_k, *recent_v;
    const float *codebook;
    const void *q;
    float *out;
    uint8_t *mask_out;
    float *part;        // partial softmax states [wave][G][D + 4]: m, l, unused x2, o[D]
    uint32_t *qprep;    // per-unit query record written by the query-prep kernel
    uint32_t *tile_ctr; // per stripe, at the place of its first member: tiles drawn [n_waves], members
                        // done [n_waves]; then per unit: members / stripes done [units]; zeroed by
                        // the query-prep kernel
    int n_kv_heads, cap, len, n_sink, rotate, ch0, keep, q_bf16;
    int n_recent;       // recent BF16 window W (0: none)
    int q_end;          // quantised positions are [n_sink, q_end); [max(n_sink, q_end), len) is the window
    float sm_log2e;      // softmax scale times log2(e)
    int n_units, tiles_per_unit, n_waves; // work split: n_waves >= n_units waves, wave w serves unit w % n_units
    int dynamic;        // 1: tiles from the unit counters; 0: member k of n takes k, k + n, ...
    int n_cu;           // compute units of the device (places of waves, see the decode kernel)
    const float *rope_cs; // bucket-relative RoPE: (cos, sin) of each bucket's anchor [bucket][D/2][2]
    int rope_lw;        // log2 of the bucket width, 0: off
    int n_rb;           // query records per unit: one per bucket of the capacity (1 without RoPE)
    int n_qb;           // buckets holding positions < len (query records the prep writes per unit)
    const float *v_codebook; // KQV values: 8 centroids
    const uint32_t *v_qjl;   // KQV values: the sketch's sign diagonal (bit set: -1)
    float *bstate;      // softmax states of the BF16 chunks [unit][bch_max][G][D + 4] (query prep)
    int n_bch;          // BF16 chunks of this call per unit: the sinks, then the window's part of
                        // each 64-aligned block of positions it touches
    int bch_max;        // chunk records per unit (1, or 2 + ceil(n_recent / 64) with a window)
};

hipError_t launch_append(int head_dim, const AppendParams &p, hipStream_t s);
// ev[0], ev[1]: optional events recorded around the decode kernel (both non-null or unused)
hipError_t launch_decode(int head_dim, int group, int kfmt, int vfmt, int units, const DecodeParams &p,
                         hipEvent_t const ev[2], hipStream_t s);
// the per-token INT2 value instantiations (compiled apart): launch, and the kernel of a shape
hipError_t launch_decode_v2(int head_dim, int group, int kfmt, int units, const DecodeParams &p,
                            hipEvent_t const ev[2], hipStream_t s);
const void *decode_kernel_v2(int head_dim, int group, int kfmt);
// the KQV value instantiations (compiled apart)
hipError_t launch_decode_v3(int head_dim, int group, int kfmt, int units, const DecodeParams &p,
                            hipEvent_t const ev[2], hipStream_t s);
const void *decode_kernel_v3(int head_dim, int group, int kfmt);
// Streaming-read probe over `bytes` (a multiple of 16) at p; out holds `blocks` words.
hipError_t launch_stream_read(const void *p, size_t bytes, uint32_t *out, int blocks, hipStream_t s);
// u32 words of one unit's query record (query-prep output read by the decode kernel).
int decode_qrec_words(int head_dim, int group, int kfmt);
// Resident decode workgroups (one wave each) the device holds for this instantiation.
int decode_slots(int head_dim, int group, int kfmt, int vfmt);
// Compute units of the current device (256 when the runtime cannot be asked).
int device_cus();
// Device address of the current device's allocation-free decode workspace
// (KVQ_NOALLOC_SCRATCH_BYTES bytes, looked up once per device).
hipError_t noalloc_scratch(void **ptr);

} // namespace kvq
