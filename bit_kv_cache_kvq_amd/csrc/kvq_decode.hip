// kvq_decode.hip -- decode attention over the packed low-bit cache: the host side of the
// decode kernels (launch, work-split queries) and the instantiations for INT4 values per
// 32-channel group.  The kernels are in kvq_decode_impl.h; kvq_decode_v2.hip and
// kvq_decode_v3.hip instantiate them for per-token INT2 and KQV values.
#include "kvq_decode_impl.h"

namespace kvq {

int decode_qrec_words(int head_dim, int group, int kfmt)
{
    return head_dim == 128 ? qrec_g<128>(group, kfmt) : qrec_g<64>(group, kfmt);
}

int device_cus()
{
    static std::atomic<int> cache{0};
    int v = cache.load();
    if (v > 0)
        return v;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0) {
        (void)hipGetLastError();
        v = 256;
    }
    cache.store(v);
    return v;
}

int decode_slots(int head_dim, int group, int kfmt, int vfmt)
{
    // resident one-wave workgroups of this instantiation on the current device, cached;
    // 256 CUs x 8 when the runtime cannot be asked (no device)
    static std::atomic<int> cache[2][4][3][3];
    const int di = head_dim == 128 ? 1 : 0;
    const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : 3;
    const int ki = kfmt < 0 ? 0 : kfmt > 2 ? 2 : kfmt;
    const int vi = vfmt == KVQ_V_ASYM2_TOKEN ? 1 : vfmt == KVQ_V_KQV ? 2 : 0;
    int v = cache[di][gi][ki][vi].load();
    if (v > 0)
        return v;
    int dev = 0, cus = 0, per_cu = 0;
    const void *k = vi == 1   ? decode_kernel_v2(head_dim, group, kfmt)
                    : vi == 2 ? decode_kernel_v3(head_dim, group, kfmt)
                              : kernel_vf<KVQ_V_ASYM4_G32>(head_dim, group, kfmt);
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kWave, 0) == hipSuccess && cus > 0 &&
        per_cu > 0) {
        v = cus * per_cu;
    } else {
        (void)hipGetLastError();
        v = 256 * 8;
    }
    cache[di][gi][ki][vi].store(v);
    return v;
}

hipError_t launch_decode(int head_dim, int group, int kfmt, int vfmt, int units, const DecodeParams &p,
                         hipEvent_t const ev[2], hipStream_t s)
{
    if (vfmt == KVQ_V_ASYM2_TOKEN)
        return launch_decode_v2(head_dim, group, kfmt, units, p, ev, s);
    if (vfmt == KVQ_V_KQV)
        return launch_decode_v3(head_dim, group, kfmt, units, p, ev, s);
    return launch_vf<KVQ_V_ASYM4_G32>(head_dim, group, kfmt, units, p, ev, s);
}

} // namespace kvq
