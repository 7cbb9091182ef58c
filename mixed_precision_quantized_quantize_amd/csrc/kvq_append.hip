// kvq_append.hip -- quantize new K/V rows into the cache planes.
//
// The quantizing row copy into the cache (the op the llama.cpp issue calls
// "CPY"), for the cache types of the llama.cpp guide's "KV-Cache-Praezision"
// section: one quad of lanes per 32-element block (the quantizer is in
// kvq_quant.h).
#include <algorithm>

#include "kvq_quant.h"

// No multiply-add contraction anywhere in this file: the q4_0 code depends
// on x*id and +8.5 being rounded separately.
#pragma clang fp contract(off)

namespace kvq {
namespace {

using namespace quant;

// K plane (token-major): one quad per (sequence, row, kv head, block); each
// lane's units are one contiguous store.
template <int KT>
__device__ inline void append_k(const AppendArgs &a, const int qd, const int q)
{
    const int NB = a.D / 32;
    const int b = qd % NB;
    int r = qd / NB;
    const int h = r % a.H;
    r /= a.H;
    const int i = r % a.n_new;
    const int s = r / a.n_new;
    const int64_t pair = (int64_t)s * a.H + h;
    const uint16_t *blk = a.src[0] + (((int64_t)s * a.n_new + i) * a.H + h) * a.D + 32 * b;
    quant_store<KT, 0>(blk, q, a.codes[0], a.scales[0], a.qh[0], pair, (int64_t)a.pos[s] + i, b, a.D, a.Tc);
}

// V plane (8-token interleaved): an item is one 8-token group of one
// (sequence, kv head) -- tokens 8g .. 8g+7 -- over all blocks.  The quad of
// (block b, token 8g+ti) quantizes and writes its units into an LDS copy of
// the group laid out as in the plane (unit u of token ti at u*8 + ti), then
// the item's threads write the group's codes, scales and bit words as whole
// 16-byte pieces.  A group only partly inside the appended range is first
// read back, so that its other tokens keep their bytes.  8/NB items per
// workgroup of 64 quads.
template <int VT>
__device__ inline void append_v(const AppendArgs &a, const int blk_id, const int tid)
{
    constexpr int W = (VT == KVQ_F16) ? 2 : 1;  // bytes per unit
    constexpr int UB = (VT == KVQ_F16) ? 32 : (int)row_code_bytes(VT, 32);  // units per block
    constexpr int NU = lane_units<VT>();
    constexpr bool BITS = VT == KVQ_Q5_0 || VT == KVQ_TURBO3;
    // staging for the 8/NB items of a workgroup: 64 (block, token) rows of UB units
    __shared__ __attribute__((aligned(16))) uint8_t st_u[64 * UB * W];
    __shared__ __attribute__((aligned(16))) uint16_t st_s[64];
    __shared__ __attribute__((aligned(16))) uint32_t st_b[64];

    const int NB = a.D / 32, IPW = 8 / NB;
    const int q = tid & 3, qw = tid >> 2;
    const int item_l = qw / (8 * NB), rem = qw - item_l * 8 * NB;
    const int b = rem >> 3, ti = rem & 7;
    // 32-bit indices: the host keeps n_seqs * H * ng below 2^31
    const int item = blk_id * IPW + item_l;
    const int n_items = a.n_seqs * a.H * a.ng;
    const int gi = item % a.ng;
    const int sh = item / a.ng;  // s * H + h
    const int s = sh / a.H;
    const bool live = item < n_items;
    const int p0 = live ? a.pos[s] : 0, p1 = p0 + a.n_new;
    const int g = p0 / 8 + gi;
    const bool exists = live && 8 * g < p1;          // the group holds an appended token
    const bool full = exists && 8 * g >= p0 && 8 * g + 8 <= p1;
    const int64_t pair = sh;
    const int64_t U = (int64_t)UB * NB;  // units per row
    const int64_t gunit = (pair * (a.Tc / 8) + g) * U * 8;  // the group's first unit in the plane
    const int64_t gscale = (pair * (a.Tc / 8) + g) * NB * 8;
    uint8_t *const stu = st_u + item_l * (8 * NB * UB * W);
    uint16_t *const sts = st_s + item_l * 8 * NB;
    uint32_t *const stb = st_b + item_l * 8 * NB;
    const int it = tid - item_l * 32 * NB;  // thread index within the item (32*NB threads)
    const int ubytes = 8 * NB * UB * W;     // the group's code bytes

    if (exists && !full) {  // read the group back: its other tokens keep their bytes
        for (int o = 16 * it; o < ubytes; o += 16 * 32 * NB)
            *reinterpret_cast<u32x4 *>(stu + o) = *reinterpret_cast<const u32x4 *>(a.codes[1] + gunit * W + o);
        if (VT != KVQ_F16 && it < 8 * NB) {
            sts[it] = a.scales[1][gscale + it];
            if (BITS)
                stb[it] = a.qh[1][gscale + it];
        }
    }
    __syncthreads();
    const int t = 8 * g + ti;
    if (exists && t >= p0 && t < p1) {
        const uint16_t *blkp = a.src[1] + (((int64_t)s * a.n_new + (t - p0)) * a.H + (pair - (int64_t)s * a.H)) * a.D + 32 * b;
        const LaneCodes lc = quant_lane<VT>(blkp, q);
#pragma unroll
        for (int k = 0; k < NU; k++) {
            const int u = UB * b + NU * q + k;  // unit within the row
            if (W == 2)
                *reinterpret_cast<uint16_t *>(stu + (u * 8 + ti) * 2) = (uint16_t)(lc.w[k >> 1] >> (16 * (k & 1)));
            else
                stu[u * 8 + ti] = (uint8_t)(lc.w[k >> 2] >> (8 * (k & 3)));
        }
        if (q == 0 && VT != KVQ_F16) {
            sts[b * 8 + ti] = lc.dbits;
            if (BITS)
                stb[b * 8 + ti] = lc.bits;
        }
    }
    __syncthreads();
    if (exists) {
        for (int o = 16 * it; o < ubytes; o += 16 * 32 * NB)
            *reinterpret_cast<u32x4 *>(a.codes[1] + gunit * W + o) = *reinterpret_cast<const u32x4 *>(stu + o);
        if (VT != KVQ_F16 && it < NB) {  // 8 scales (16 B) and 8 bit words (32 B) per block
            *reinterpret_cast<u32x4 *>(a.scales[1] + gscale + 8 * it) = *reinterpret_cast<const u32x4 *>(sts + 8 * it);
            if (BITS) {
                *reinterpret_cast<u32x4 *>(a.qh[1] + gscale + 8 * it) = *reinterpret_cast<const u32x4 *>(stb + 8 * it);
                *reinterpret_cast<u32x4 *>(a.qh[1] + gscale + 8 * it + 4) = *reinterpret_cast<const u32x4 *>(stb + 8 * it + 4);
            }
        }
    }
}

// blockIdx.y = 0: K plane (n_quads quads, 64 per workgroup); 1: V plane
// (8-token groups, 8/NB per workgroup).  Workgroups past a role's work leave
// together, before any barrier.
template <int KT, int VT>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a, int n_quads, int v_blocks)
{
    if (blockIdx.y == 0) {
        const int qd = blockIdx.x * 64 + (threadIdx.x >> 2);
        if (qd < n_quads)  // whole quads leave together: the shuffles stay inside a quad
            append_k<KT>(a, qd, threadIdx.x & 3);
    } else if ((int)blockIdx.x < v_blocks) {
        append_v<VT>(a, blockIdx.x, threadIdx.x);
    }
}

template <int KT, int VT>
hipError_t launch_t(const AppendArgs &a, int n_quads, hipStream_t st)
{
    const int NB = a.D / 32, IPW = 8 / NB;
    const int64_t n_items = (int64_t)a.n_seqs * a.H * a.ng;
    const int v_blocks = (int)((n_items + IPW - 1) / IPW);
    const int k_blocks = (n_quads + 63) / 64;
    dim3 grid(std::max(k_blocks, v_blocks), 2);
    hipLaunchKernelGGL((append_kernel<KT, VT>), grid, dim3(256), 0, st, a, n_quads, v_blocks);
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
