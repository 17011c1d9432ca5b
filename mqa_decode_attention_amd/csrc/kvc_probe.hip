// kvc_probe.hip - streaming-read probe: the HBM read bandwidth a plain kernel
// reaches on this device, the practical ceiling for a read-bound kernel such
// as decode attention.  Each workgroup reads one contiguous slice with 16-byte
// loads, 16 in flight per thread, and folds the data into one word so that
// nothing is optimised away.  The loads use the default cache policy or the
// non-temporal one (the policy of the decode kernels' K/V loads).

#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kProbeUnroll = 16;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ void __launch_bounds__(256) read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                         size_t per_wg, unsigned* sink) {
    const size_t beg = static_cast<size_t>(blockIdx.x) * per_wg;
    const size_t end = beg + per_wg < n16 ? beg + per_wg : n16;
    unsigned acc = 0;
    for (size_t i = beg + threadIdx.x; i < end; i += 256 * kProbeUnroll) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const size_t k = i + static_cast<size_t>(u) * 256;
            if (k < end)
                v[u] = NT ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + k)))
                          : src[k];
            else v[u] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;   // practically never taken
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, unsigned* sink, int workgroups,
                             bool nontemporal, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const size_t per = (n16 + workgroups - 1) / workgroups;
    if (nontemporal)
        hipLaunchKernelGGL(read_probe_kernel<true>, dim3(workgroups), dim3(256), 0, stream,
                           static_cast<const uint4*>(buf), n16, per, sink);
    else
        hipLaunchKernelGGL(read_probe_kernel<false>, dim3(workgroups), dim3(256), 0, stream,
                           static_cast<const uint4*>(buf), n16, per, sink);
    return hipGetLastError();
}

}  // namespace kvc
