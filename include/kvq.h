/*
 * kvq.h -- C ABI of libkvq: low-bit quantized KV-cache append and decode attention on
 * AMD MI355X (gfx950).
 *
 * The method (sources are the pages this library implements; sections as they name them):
 *   - Keys: optionally Walsh-Hadamard-rotated, then either asymmetric INT2/INT4 with an
 *     FP16 scale and zero per 32-channel group, channel 0 optionally kept in BF16 and left
 *     out of the range estimate (Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit
 *     KV Caches, sec. 3.3 and C.3), or 4-bit codes of an N(0,1) Lloyd-Max codebook with an
 *     FP16 per-vector norm (TurboQuant on Quantized Models: abstract and topic list;
 *     Statistical Inference and Quality Measures of KV Cache Quantisations Inspired by
 *     TurboQuant: scheme KQV and the Beta -> Gaussian marginal).
 *   - Keys stored channel-major so decode reads only the channel rows it keeps
 *     (Dual-QK sec. 3.3).
 *   - Values: asymmetric INT4 with an FP16 scale and zero per 32-channel group, or
 *     per-token asymmetric INT2 with a clipping ratio and one FP16 scale and zero per token
 *     (Dual-QK sec. 3.3 and B.2: per-token INT2 values with a 0.92 clipping ratio), or
 *     KQV's value side: Walsh-Hadamard-rotated values as 3-bit Lloyd-Max codes with an FP16
 *     norm plus a 1-bit QJL sketch of the residual through a randomised Hadamard transform,
 *     4 bits per channel in all (Statistical Inference and Quality Measures of KV Cache
 *     Quantisations Inspired by TurboQuant: scheme KQV and the QJL estimator; TurboQuant on
 *     Quantized Models, abstract: SRHT-QJL).
 *   - The first n_sink positions of every sequence are stored in BF16 (TurboQuant on
 *     Quantized Models, abstract: sink-token preservation; Dual-QK sec. 3.3 / 4.1), and
 *     optionally the n_recent most recent ones too, quantized only when they leave that
 *     window (Dual-QK sec. 3.3 / 4.1: the most recent 256 entries stay BF16; TurboQuant on
 *     Quantized Models, abstract: past-only quantization).
 *   - Decode scores queries straight against the packed codes (TurboQuant on Quantized
 *     Models, abstract: fused scoring without key decompression), with optional dynamic
 *     query-channel-group pruning: one mask per GQA group keeping the m 16-channel groups
 *     of largest query energy summed over the group's heads (Dual-QK sec. 3.2, C.2,
 *     App. A), and one softmax over all positions (Dual-QK sec. 3.4).
 *   - Optional bucket-relative RoPE (Dual-QK sec. 3.4 and C.4): keys arrive with their
 *     rotary embedding applied at their absolute position t and are stored relative to the
 *     anchor a = w * floor(t / w) of their bucket (w = rope_bucket), i.e. rotated back by a;
 *     decode rotates the query back by each bucket's anchor before scoring that bucket, so
 *     every score equals the one of the un-bucketed keys before quantization.  The masks may
 *     differ across buckets; all buckets share one softmax.
 *
 * Conventions for every entry point:
 *   - All buffer pointers are DEVICE pointers owned by the caller unless stated otherwise.
 *     The library never allocates device memory and never synchronizes; all work is
 *     enqueued on the caller's stream (`stream` is a hipStream_t, NULL = null stream).
 *   - Arguments are validated on the host before anything is enqueued; on any error code
 *     other than KVQ_ERR_HIP nothing was launched and the cache is unchanged.
 *   - Calls on distinct caches are thread-safe; calls on one cache must be ordered.
 *
 * Packed layout (U = batch * n_kv_heads units; unit u = b * n_kv_heads + kv_head; every
 * array is indexed by absolute token position t in [0, capacity)):
 *   k_codes  u32 [U][R][capacity]  R = head_dim/16 (INT2) or head_dim/8 (4-bit).  Word
 *                                  (r, t) holds channels r*(32/b) .. r*(32/b)+32/b-1 of
 *                                  token t, channel r*(32/b)+j in bits [b*j, b*j+b-1].
 *   k_sz     u32 [U][head_dim/32][capacity]  asymmetric keys: fp16 scale in bits 0-15,
 *                                  fp16 zero (the group minimum) in bits 16-31.
 *   k_norm   u16 [U][capacity]     Lloyd-Max keys: fp16 norm rho (RMS of the stored
 *                                  coordinates; equals ||k|| when rotated).
 *   k_ch0    u16 [U][capacity]     protected channel 0: bf16.
 *   v_codes  u32 [U][capacity/2][head_dim/4]  INT4 values: word j of token pair P holds
 *                                  channels 4j..4j+3: token 2P in bits 0-15, token 2P+1 in
 *                                  bits 16-31, channel 4j+k at nibble k of its half.
 *            u32 [U][capacity/2][head_dim/8]  per-token INT2 values: word j of pair P holds
 *                                  channels 8j..8j+7, token 2P in bits 0-15, token 2P+1 in
 *                                  bits 16-31, channel 8j+k at bits [2k, 2k+1] of its half.
 *            KQV values use the INT4 layout; nibble i = 3-bit code | sketch bit << 3.
 *   v_sz     u32 [U][head_dim/32][capacity]  INT4 values: fp16 scale | fp16 zero << 16 per
 *                                  group; per-token INT2 values: [U][1][capacity]; KQV values:
 *                                  [U][1][capacity], fp16 norm rho | fp16 residual norm << 16.
 *   v_codebook f32 [8], v_thresholds f32 [7]  KQV values: the 8-level N(0,1) Lloyd-Max
 *                                  centroids ascending and their thresholds.
 *   v_qjl_signs u32 [head_dim/32]  KQV values: the sketch's random sign diagonal D (bit i set:
 *                                  channel i negated), drawn once by the caller.
 *   sink_k   u16 [U][n_sink][head_dim]  bf16 keys of positions < n_sink, in stored
 *                                  coordinates (rotated when k_hadamard = 1).
 *   sink_v   u16 [U][n_sink][head_dim]  bf16 values of positions < n_sink.
 *   recent_k u16 [U][n_recent][head_dim]  recent window (n_recent = W > 0): ring slot t mod
 *   recent_v u16 [U][n_recent][head_dim]  W holds the bf16 key (stored coordinates) / value
 *                                  of position t while t is one of the W most recent
 *                                  positions >= n_sink.
 *   rope_cs  f32 [ceil(capacity / rope_bucket)][head_dim/2][2]  bucket-relative RoPE: entry
 *                                  (b, i) = (cos, sin) of the anchor b*w times the model's
 *                                  rotary frequency of channel pair i (its checkpoint's
 *                                  frequencies, scaled ones included); filled by the caller.
 *   codebook f32 [16], thresholds f32 [15]  Lloyd-Max keys: centroids ascending and the
 *                                  decision thresholds; a rotated coordinate z codes to the
 *                                  number of thresholds strictly below z.
 * Quantized arrays are never written or read at positions t < n_sink, nor at positions still
 * in the recent window; with a window, a position is quantized from its bf16 copy (keys in
 * stored coordinates) when it leaves the window, so its codes do not depend on how the
 * appends were cut.
 * Encoding arithmetic is fixed (fp32, IEEE round-to-nearest-even, no contraction) so the
 * packed bytes are reproducible bit for bit:
 *   asym b-bit group: scale = fp16((max - min) / (2^b - 1)), zero = fp16(min), with
 *   channel 0 excluded from min/max when protected; code = clamp(rint((x - zero) *
 *   (scale > 0 ? 1/scale : 0)), 0, 2^b - 1) using the fp16-rounded scale and zero.
 *   Lloyd-Max: y = FWHT(k) (unnormalised, stages h = 1, 2, 4, ... writing (a+b, a-b)) when
 *   rotated, else y = k; rho = fp16(sqrt(tree_sum(y*y) / d)) with the stride-halving
 *   tree; z = y * (rho > 0 ? 1/rho : 0).
 *   per-token INT2 values: the range is clipped to [c*min, c*max] (c = v_clip, both ends
 *   scaled toward zero), scale = fp16((c*max - c*min) / 3), zero = fp16(c*min), codes as
 *   for the asymmetric groups (entries outside the clipped range saturate at 0 or 3).
 *   KQV values: y = FWHT(v), rho as for Lloyd-Max keys, code = number of the 7 thresholds
 *   strictly below y * (1/rho), r = y - rho * cent[code], sketch bit i = 1 when
 *   (FWHT(D r))_i < 0, residual norm = fp16(sqrt(tree_sum(r*r))).  Decode reads
 *   v^ = FWHT(rho cent[code] + sqrt(pi/2)/d * ||r|| * D FWHT(sigma)) / d, sigma_i = -1 for
 *   a set bit (the QJL estimator with S = FWHT * D).
 *   bucket-relative RoPE (rotate-half pairing: channel i pairs with i + head_dim/2): with
 *   (c, s) = rope_cs[t / w][i], k'_i = k_i*c + k_{i+d/2}*s and k'_{i+d/2} = k_{i+d/2}*c -
 *   k_i*s (each product rounded, then the sum), before the Walsh-Hadamard rotation.  The
 *   decode query of bucket b is rotated the same way with entry b.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_ARG = -1,         /* null pointer, bad size or out-of-range argument       */
    KVQ_ERR_UNSUPPORTED = -2, /* valid but unsupported combination (e.g. head_dim 96)   */
    KVQ_ERR_CAPACITY = -3,    /* len + n_new > capacity                                 */
    KVQ_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required             */
    KVQ_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                       */
    KVQ_ERR_HIP = -6          /* a kernel launch failed; appended range is undefined    */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;

typedef enum { KVQ_K_ASYM2 = 0, KVQ_K_ASYM4 = 1, KVQ_K_LLOYD4 = 2 } kvq_kfmt;

typedef enum { KVQ_V_ASYM4_G32 = 0, KVQ_V_ASYM2_TOKEN = 1, KVQ_V_KQV = 2 } kvq_vfmt;

/* Cache descriptor.  Geometry and format fields are set once by the caller; `len` is the
 * number of positions stored per sequence (uniform across sequences) and is advanced by
 * kvq_quant_append.  Constraints: head_dim in {64, 128}; capacity a positive multiple of
 * 256 and at most 2^24; batch * n_kv_heads <= 65535; 0 <= n_sink <= 64 and n_sink < capacity; k_hadamard and k_ch0_bf16 in {0, 1};
 * k_ch0_bf16 requires an asymmetric key format and k_hadamard = 0; v_format is a
 * kvq_vfmt, and v_clip (per-token INT2 values only, otherwise ignored) lies in (0, 1];
 * 0 <= n_recent <= 1024; rope_bucket is 0 (off) or a power of two in [128, 2^24], and needs
 * rope_cs.
 * Pointers unused by the chosen format may be NULL (see kvq_buffer_bytes).              */
typedef struct kvq_cache {
    int32_t batch, n_kv_heads, head_dim, capacity, n_sink;
    int32_t k_format, k_hadamard, k_ch0_bf16;
    int32_t len;
    uint32_t *k_codes;
    uint32_t *k_sz;
    uint16_t *k_norm;
    uint16_t *k_ch0;
    uint32_t *v_codes;
    uint32_t *v_sz;
    uint16_t *sink_k;
    uint16_t *sink_v;
    const float *codebook;
    const float *thresholds;
    int32_t v_format;
    float v_clip;
    int32_t n_recent;
    uint16_t *recent_k;
    uint16_t *recent_v;
    int32_t rope_bucket;
    const float *rope_cs;
    const float *v_codebook;
    const float *v_thresholds;
    const uint32_t *v_qjl_signs;
} kvq_cache;

enum {
    KVQ_BUF_K_CODES = 0,
    KVQ_BUF_K_SZ = 1,
    KVQ_BUF_K_NORM = 2,
    KVQ_BUF_K_CH0 = 3,
    KVQ_BUF_V_CODES = 4,
    KVQ_BUF_V_SZ = 5,
    KVQ_BUF_SINK_K = 6,
    KVQ_BUF_SINK_V = 7,
    KVQ_BUF_CODEBOOK = 8,
    KVQ_BUF_THRESHOLDS = 9,
    KVQ_BUF_RECENT_K = 10,
    KVQ_BUF_RECENT_V = 11,
    KVQ_BUF_ROPE_CS = 12,
    KVQ_BUF_V_CODEBOOK = 13,
    KVQ_BUF_V_THRESHOLDS = 14,
    KVQ_BUF_V_QJL_SIGNS = 15
};

/* Bytes the caller must allocate for buffer `which` (KVQ_BUF_*) of this geometry; 0 when
 * the format does not use that buffer or the geometry is invalid.  Host-only, no HIP.    */
size_t kvq_buffer_bytes(const kvq_cache *c, int32_t which);

/* Host-side check of a descriptor (geometry, format flags, pointers and their 16-byte
 * alignment, 0 <= len <= capacity).  Returns KVQ_OK or the first error found.             */
kvq_status kvq_validate(const kvq_cache *c);

/* Numerical domain (what the parity tests cover).  Every stored parameter is an fp16, so
 * inputs must be finite with |x| < 65504 in stored coordinates (see kvq_quant_append), and
 * the parameters that are norms must stay below
 * 65504 too: Lloyd-Max keys need ||k||_2 < 65504 (rho is the key's L2 norm when rotated),
 * KQV values need ||v||_2 below about 3e4 (their residual norm is about 2.1 ||v||_2 at
 * head_dim 128).  Decode scores the query as fp16 halves of the query before the softmax
 * scale (a power-of-two scale puts the largest kept |q| in [2^12, 2^13)): a bf16 query over
 * unrotated keys is carried exactly, any other keeps 11 bits relative to each channel.  A
 * sharp query -- some head's largest |q_c| above 8 times its fifth largest, in the
 * coordinates the query is given in -- also takes each channel's residual half (about 22
 * bits), and Lloyd-Max centroids their fp16 residuals.  Value weights p * s (p the softmax
 * weight, s a value scale or KQV norm) are fp16 products carrying a running power of two per
 * decode wave, lowered whenever a larger scale arrives, so any finite scale is supported; a
 * scale more than 2^26 below the largest one a wave has met earlier loses relative precision
 * (its weights become fp16 subnormals).  Within this domain, outputs stay within 2e-3 of the
 * row norm of exact attention over the decoded cache for logits of moderate size (the error
 * of a logit grows with sm * sum_c |q_c k_c|, which also grows the softmax's sensitivity).  */

/* Append n_new tokens to every sequence: quantize and pack k_new / v_new
 * ([batch][n_kv_heads][n_new][head_dim], dtype KVQ_F32 or KVQ_BF16, row-major, device)
 * into positions [len, len + n_new), then set len += n_new.  Only those positions are
 * written (O(1) work per appended token; TurboQuant on Quantized Models, abstract:
 * incremental cache).  Positions below n_sink go to sink_k / sink_v in BF16.  With a
 * recent window, new positions go to the ring in BF16 and the positions leaving the window
 * (old ones, and new ones already W behind the new end) are quantized from their BF16
 * copies; this takes two kernel launches, eviction first.  Inputs must be finite with
 * |x| < 65504 in stored coordinates so the fp16 parameters stay finite (the anchor rotation
 * of bucket-relative RoPE can grow an entry by up to sqrt(2), and the unnormalised
 * Walsh-Hadamard rotation of asymmetric keys by up to head_dim); other inputs give
 * unspecified codes.  n_new = 0 is a no-op.                                               */
kvq_status kvq_quant_append(kvq_cache *c, const void *k_new, const void *v_new, int32_t dtype,
                            int32_t n_new, void *stream);

/* Workspace bytes kvq_decode_attn needs for this cache geometry (any len up to capacity)
 * and n_q_heads.  The workspace holds the query records (one per sequence, KV head and RoPE
 * bucket), the partial softmax states of the decode waves, the softmax states of the BF16
 * positions (sinks and recent window) and the tile and arrival counters; its contents need
 * no initialisation and are scratch between calls.                                         */
size_t kvq_decode_workspace_bytes(const kvq_cache *c, int32_t n_q_heads);

/* Decode attention for one query step per sequence over positions [0, len).
 *   q        [batch][n_q_heads][head_dim], KVQ_F32 or KVQ_BF16, device.  n_q_heads must be
 *            a multiple of n_kv_heads with G = n_q_heads / n_kv_heads in {1, 2, 4, 8};
 *            query head h reads KV head floor(h / G).
 *   sm_scale softmax scale applied to q.k (1/sqrt(head_dim) for standard attention).
 *   keep_groups  m: keep the m 16-channel groups of largest summed query energy (ties to
 *            the lower group), 0 or >= head_dim/16 keeps all channels.  The mask applies to
 *            every key (sink tokens included) and never to values.
 *   out      [batch][n_q_heads][head_dim] fp32, device.
 *   mask_out nullable, [batch * n_kv_heads] bytes, bit p set = group p was read.  With
 *            bucket-relative RoPE: [batch * n_kv_heads][ceil(capacity / rope_bucket)] bytes,
 *            entry (u, b) the mask of bucket b, written for b < ceil(len / rope_bucket).
 *   q        with bucket-relative RoPE: the query with its rotary embedding applied at its
 *            own position (as the keys were when appended).
 *   ws       workspace of ws_bytes >= kvq_decode_workspace_bytes(c, n_q_heads).
 * len = 0 writes zeros.  By default the waves serving one sequence and KV head take its
 * 128-position tiles in the order they ask for them, so the fp32 summation order, and the
 * last bits of out, can differ between calls; kvq_set_deterministic(1) fixes the order.   */
kvq_status kvq_decode_attn(const kvq_cache *c, const void *q, int32_t q_dtype, int32_t n_q_heads,
                           float sm_scale, int32_t keep_groups, float *out, uint8_t *mask_out,
                           void *ws, size_t ws_bytes, void *stream);

/* Allocation-free decode, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same as
 * kvq_decode_attn -- same kernels, outputs, masks, status codes and argument checks -- but
 * the workspace is a device-resident array of KVQ_NOALLOC_SCRATCH_BYTES bytes inside the
 * library, one per GPU, held until the process ends.  A call needs
 * kvq_decode_noalloc_scratch_bytes(c, n_q_heads) bytes of it (the partial states of the
 * waves this call launches, the query records and the counters); beyond the array's size it
 * returns KVQ_ERR_WORKSPACE before anything is enqueued.  Nothing is allocated: the array's
 * device address is looked up once per device (on the first call with that device
 * current), and the query-prep kernel clears the counters on every call.  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller.                                              */
#define KVQ_NOALLOC_SCRATCH_BYTES (32u << 20)
kvq_status kvq_decode_attn_noalloc(const kvq_cache *c, const void *q, int32_t q_dtype, int32_t n_q_heads,
                                   float sm_scale, int32_t keep_groups, float *out, uint8_t *mask_out,
                                   void *stream);
/* Bytes of the array one kvq_decode_attn_noalloc call of this geometry, len and n_q_heads
 * needs; 0 for an invalid geometry.  Host-only apart from querying the device's occupancy
 * once.                                                                                   */
size_t kvq_decode_noalloc_scratch_bytes(const kvq_cache *c, int32_t n_q_heads);

/* Number of decode waves kvq_decode_attn uses for the current len: one per resident wave
 * slot of the device, at most one per 128-position tile and at least one per (sequence,
 * KV head); wave w serves (sequence, KV head) number w mod (batch * n_kv_heads).  Host-only
 * apart from querying the device's occupancy once.                                       */
int32_t kvq_decode_splits(const kvq_cache *c, int32_t n_q_heads);

/* Host helper: the 2^bits-level symmetric Lloyd-Max codebook of N(0,1) (fp64 Newton
 * iteration on the decision boundaries, rounded to fp32), written to HOST arrays
 * centroids[2^bits], thresholds[2^bits-1] (the centroids' midpoints); 1 <= bits <= 6.
 * bits = 4 serves the Lloyd-Max keys and bits = 3 the KQV values.                         */
kvq_status kvq_codebook_gaussian(int32_t bits, float *centroids, float *thresholds);

/* Tuning override for the work split: target number of 128-position tiles per decode wave,
 * 0 = the built-in policy (one wave per resident slot).  Process-wide; affects later
 * decode calls only.                                                                     */
void kvq_set_split_tiles(int32_t tiles_per_split);

/* 1: every decode wave takes a fixed set of tiles (member k of a team of n waves takes the
 * k-th of n contiguous shares of its stripe's tiles), so kvq_decode_attn gives bit-identical
 * outputs for identical inputs; 0 (default): the first three quarters of a stripe's tiles
 * are shared that way and the rest go to whichever wave of the team asks first, which
 * balances waves that get unequal shares of their SIMD.  Process-wide; affects later calls
 * only.                                                                                  */
void kvq_set_deterministic(int32_t on);

/* Measurement hook: while both handles are non-NULL (hipEvent_t, created and owned by the
 * caller), every kvq_decode_attn launches its main decode kernel with start_event and
 * stop_event attached to the dispatch (hipExtLaunchKernel): they record the start and the
 * end of that kernel's execution, so hipEventElapsedTime gives its duration alone (the
 * query-prep kernel falls outside).  NULL, NULL turns it off.  Process-wide; meant for
 * benchmarks, not for concurrent callers.                                                 */
void kvq_set_decode_events(void *start_event, void *stop_event);

/* Measurement probe: reads `bytes` of device memory at `p` once and writes one XOR word per
 * workgroup to `out` (device, `blocks` u32): `blocks` one-wave workgroups each read one
 * contiguous share with 16-byte non-temporal loads (1 KiB per wave and instruction, 8 in
 * flight), the way decode waves read their units' tiles.  Its rate is the practical HBM
 * read ceiling the decode kernel is compared with.  bytes must be a positive multiple of
 * 16, p and out 16-byte aligned, 1 <= blocks <= 65535.                                   */
kvq_status kvq_probe_stream_read(const void *p, size_t bytes, uint32_t *out, int32_t blocks, void *stream);

const char *kvq_status_string(kvq_status s);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
