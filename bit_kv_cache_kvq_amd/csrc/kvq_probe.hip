// kvq_probe.hip -- streaming-read probe: the practical HBM read rate of this device, the
// ceiling the decode kernel's effective bandwidth is compared with (besides the 8 TB/s
// peak).  Each one-wave workgroup reads one contiguous share of the buffer once, as a
// decode wave reads its unit's tiles: 16-byte non-temporal loads, a 1 KiB row per wave and
// instruction, 8 rows in flight.  The words are folded into one XOR per workgroup so the
// reads cannot be dropped.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef unsigned int u4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kWave) void stream_read_kernel(const u4v *__restrict__ p, size_t n16,
                                                            uint32_t *__restrict__ out)
{
    constexpr int U = 8; // rows of 64 words in flight per wave
    const size_t b = blockIdx.x, nb = gridDim.x;
    const size_t lo = b * n16 / nb, hi = (b + 1) * n16 / nb; // this wave's words
    const int lane = threadIdx.x;
    u4v acc = {0u, 0u, 0u, 0u};
    size_t i = lo + (size_t)lane;
    for (; i + (U - 1) * kWave < hi; i += U * kWave) {
        u4v v[U];
#pragma unroll
        for (int j = 0; j < U; j++)
            v[j] = __builtin_nontemporal_load(p + i + j * kWave);
#pragma unroll
        for (int j = 0; j < U; j++)
            acc ^= v[j];
    }
    for (; i < hi; i += kWave)
        acc ^= __builtin_nontemporal_load(p + i);
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x ^= (uint32_t)__shfl_xor((int)x, m);
    if (lane == 0)
        out[b] = x;
}

} // namespace

hipError_t launch_stream_read(const void *p, size_t bytes, uint32_t *out, int blocks, hipStream_t s)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kWave), 0, s,
                       static_cast<const u4v *>(p), bytes / 16, out);
    return hipGetLastError();
}

} // namespace kvq
