// kvq_append.hip -- quantize new K/V rows into the cache planes.
//
// The quantizing row copy into the cache (the op the llama.cpp issue calls
// "CPY"), for the cache types of the llama.cpp guide's "KV-Cache-Praezision"
// section: one quad of lanes per 32-element block (the quantizer is in
// kvq_quant.h).
#include "kvq_quant.h"

// No multiply-add contraction anywhere in this file: the q4_0 code depends
// on x*id and +8.5 being rounded separately.
#pragma clang fp contract(off)

namespace kvq {
namespace {

using namespace quant;

template <int KT, int VT>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a, int n_quads)
{
    const int qd = blockIdx.x * 64 + (threadIdx.x >> 2);
    const int q = threadIdx.x & 3;
    if (qd >= n_quads)
        return;  // whole quads leave together: the shuffles stay inside a quad
    const int NB = a.D / 32;
    const int b = qd % NB;
    int r = qd / NB;
    const int h = r % a.H;
    r /= a.H;
    const int i = r % a.n_new;
    const int s = r / a.n_new;
    const int64_t pair = (int64_t)s * a.H + h;
    const int64_t t = (int64_t)a.pos[s] + i;
    const int role = blockIdx.y;
    const uint16_t *blk = a.src[role] + (((int64_t)s * a.n_new + i) * a.H + h) * a.D + 32 * b;
    if (role == 0)
        quant_store<KT, 0>(blk, q, a.codes[0], a.scales[0], a.qh[0], pair, t, b, a.D, a.Tc);
    else
        quant_store<VT, 1>(blk, q, a.codes[1], a.scales[1], a.qh[1], pair, t, b, a.D, a.Tc);
}

template <int KT, int VT>
hipError_t launch_t(const AppendArgs &a, int n_quads, hipStream_t st)
{
    dim3 grid((n_quads + 63) / 64, 2);
    hipLaunchKernelGGL((append_kernel<KT, VT>), grid, dim3(256), 0, st, a, n_quads);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int kt, int vt, const AppendArgs &a, int n_quads, hipStream_t st)
{
#define KVQ_A(K, V) \
    if (kt == K && vt == V) return launch_t<K, V>(a, n_quads, st);
    KVQ_FOR_EACH_TYPE_PAIR(KVQ_A)
#undef KVQ_A
    return hipErrorInvalidValue;
}

}  // namespace kvq
