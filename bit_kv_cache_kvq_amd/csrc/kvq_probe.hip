// kvq_probe.hip -- streaming-read probe: the practical HBM read rate of this device, the
// ceiling the decode kernel's effective bandwidth is compared with (besides the 8 TB/s
// peak).  Every 16-byte word is read once with non-temporal loads by a grid-stride loop;
// the words are folded into one XOR per block so the reads cannot be dropped.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef unsigned int u4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kBlock) void stream_read_kernel(const u4v *__restrict__ p, size_t n16,
                                                             uint32_t *__restrict__ out)
{
    constexpr int U = 8; // independent loads in flight per thread
    const size_t stride = (size_t)gridDim.x * kBlock;
    size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
    u4v acc = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u4v v[U];
#pragma unroll
        for (int j = 0; j < U; j++)
            v[j] = __builtin_nontemporal_load(p + i + j * stride);
#pragma unroll
        for (int j = 0; j < U; j++)
            acc ^= v[j];
    }
    for (; i < n16; i += stride)
        acc ^= __builtin_nontemporal_load(p + i);
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    __shared__ uint32_t red[kBlock];
    red[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < kBlock; t++)
            r ^= red[t];
        out[blockIdx.x] = r;
    }
}

} // namespace

hipError_t launch_stream_read(const void *p, size_t bytes, uint32_t *out, int blocks, hipStream_t s)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                       static_cast<const u4v *>(p), bytes / 16, out);
    return hipGetLastError();
}

} // namespace kvq
