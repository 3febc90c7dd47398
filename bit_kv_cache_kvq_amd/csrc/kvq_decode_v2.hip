// kvq_decode_v2.hip -- the decode kernels instantiated for per-token INT2 values (Dual-QK:
// Sharp Queries and Flat Keys for Prunable 2-bit KV Caches, sec. B.2), compiled apart from
// the INT4 ones so the two builds run in parallel.  Kernels: kvq_decode_impl.h.
#include "kvq_decode_impl.h"

namespace kvq {

hipError_t launch_decode_v2(int head_dim, int group, int kfmt, int units, const DecodeParams &p,
                            hipEvent_t const ev[2], hipStream_t s)
{
    return launch_vf<KVQ_V_ASYM2_TOKEN>(head_dim, group, kfmt, units, p, ev, s);
}

const void *decode_kernel_v2(int head_dim, int group, int kfmt)
{
    return kernel_vf<KVQ_V_ASYM2_TOKEN>(head_dim, group, kfmt);
}

} // namespace kvq
