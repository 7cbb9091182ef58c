// kvq_probe.hip -- measurement support: a plain streaming read of device
// memory, the practical bandwidth ceiling that the decode's HBM figures are
// compared with.  Not part of the attention path.
//
// Every workgroup streams one contiguous share of the buffer, each lane
// keeping eight 16-byte non-temporal loads in flight (the decode's copies
// use the same streaming cache policy), and folds them with XOR, so the loads are not removed; the fold is written
// only if it equals a value the caller passes (a store that practically never
// happens, so the kernel's traffic is reads only).
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "kvq.h"
#include "kvq_probe.h"

namespace kvq {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 8;

__global__ __launch_bounds__(PROBE_THREADS) void stream_read_kernel(const v4u *src, size_t n16, size_t chunk16,
                                                                    uint32_t key, uint32_t *sink)
{
    // workgroup b reads elements [b*chunk16, (b+1)*chunk16): each load
    // instruction of a wave covers 1 KB, one round of the workgroup 32 KB,
    // all contiguous
    const size_t begin = (size_t)blockIdx.x * chunk16;
    const size_t end = begin + chunk16 < n16 ? begin + chunk16 : n16;
    size_t i = begin + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (PROBE_UNROLL - 1) * PROBE_THREADS < end; i += PROBE_UNROLL * PROBE_THREADS) {
        v4u v[PROBE_UNROLL];
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; u++)
            v[u] = __builtin_nontemporal_load(src + i + u * PROBE_THREADS);
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; u++)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += PROBE_THREADS) {
        const v4u v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == key)
        sink[0] = acc;
}

}  // namespace
}  // namespace kvq

extern "C" int kvq_stream_read(const void *src, size_t bytes, uint32_t key, uint32_t *sink, int32_t blocks,
                               void *stream)
{
    if (!src || !sink || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 || blocks < 0)
        return KVQ_E_ARG;
    if (bytes == 0)
        return KVQ_OK;
    int nb = blocks;
    if (nb == 0) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        nb = 8 * cus;  // eight workgroups of 256 threads per CU
    }
    const size_t n16 = bytes / 16, round = (size_t)kvq::PROBE_THREADS * kvq::PROBE_UNROLL;
    const size_t chunk16 = ((n16 + nb - 1) / nb + round - 1) / round * round;  // whole rounds per workgroup
    hipLaunchKernelGGL(kvq::stream_read_kernel, dim3(nb), dim3(kvq::PROBE_THREADS), 0, (hipStream_t)stream,
                       (const kvq::v4u *)src, n16, chunk16, key, sink);
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_E_HIP;
}
