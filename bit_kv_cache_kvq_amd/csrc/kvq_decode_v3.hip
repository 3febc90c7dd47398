// kvq_decode_v3.hip -- the decode kernels instantiated for KQV values (Walsh-Hadamard-rotated
// 3-bit Lloyd-Max codes plus a 1-bit QJL sketch of the residual; Statistical Inference and
// Quality Measures of KV Cache Quantisations Inspired by TurboQuant, scheme KQV), compiled
// apart from the other value formats so the builds run in parallel.  Kernels:
// kvq_decode_impl.h.
#include "kvq_decode_impl.h"

namespace kvq {

hipError_t launch_decode_v3(int head_dim, int group, int kfmt, int units, const DecodeParams &p,
                            hipEvent_t const ev[2], hipStream_t s)
{
    return launch_vf<KVQ_V_KQV>(head_dim, group, kfmt, units, p, ev, s);
}

const void *decode_kernel_v3(int head_dim, int group, int kfmt)
{
    return kernel_vf<KVQ_V_KQV>(head_dim, group, kfmt);
}

} // namespace kvq
