// kvq_decode.hip -- split-K flash decode over the quantized cache, then a
// log-sum-exp merge of the split partials.
//
// Flash attention in the sense of the llama.cpp guide's "Flash Attention"
// section (tiled, the score matrix never materialized, exactly softmax
// attention), reading the quantized blocks directly as the KVSplit page's
// discussion asks ("integrated directly into FlashAttention") -- the
// quantized-V-requires-flash-attention rule of the llama.cpp issue.
//
// One workgroup = (split of the context, kv head, sequence), four waves.
// Each wave walks 32-token tiles of the split and serves the whole GQA group
// (up to 16 query heads) of its kv head with two matrix-core contractions
// per tile, both v_mfma_f32_16x16x32_f16:
//   S^T[token][head] = K[token][c] . Q^T[c][head]   (one MFMA per 16 tokens
//       and 32-channel block: the raw codes are exact in binary16, the
//       block's K scale is applied to the MFMA result per token)
//   O^T[chan][head] += V^T[chan][token] . P'[token][head]  (one MFMA per
//       16 channels and 32 tokens; P' = p * (V scale of that token and
//       block), rounded once to binary16)
// The score layout of the first product is exactly the operand layout the
// second one needs, so probabilities never leave registers.  The V plane is
// stored 8 tokens interleaved so each lane's P.V operand (8 tokens of one
// channel) is a single 8- or 16-byte load.  Online softmax runs in base 2
// (scores pre-multiplied by scale*log2 e).  The four waves' (m, l, O) merge
// in LDS and the workgroup writes one partial per (query head, split).
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr int TILE = 32;

__device__ inline floatx4 mfma(half8 a, half8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline half2 bits_h2(uint32_t w) { return __builtin_bit_cast(half2, w); }
__device__ inline uint32_t h2_bits(half2 h) { return __builtin_bit_cast(uint32_t, h); }

__device__ inline half8 pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(half8, v);
}

// 8 int8 codes -> 8 exact binary16 values.  Bytes are biased to unsigned,
// placed under the exponent pattern 0x64 (binary16 1024 + u), then 1152 is
// subtracted: exact for every code.
__device__ inline half8 deq_q8(u32x2 w)
{
    const uint32_t x0 = w.x ^ 0x80808080u, x1 = w.y ^ 0x80808080u;
    const half2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    uint32_t r0 = h2_bits(bits_h2(__builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u)) - off);
    uint32_t r1 = h2_bits(bits_h2(__builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u)) - off);
    uint32_t r2 = h2_bits(bits_h2(__builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u)) - off);
    uint32_t r3 = h2_bits(bits_h2(__builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)) - off);
    return pack4(r0, r1, r2, r3);
}

// 4-bit fields at bit offsets sh and sh+16 -> binary16 pair (c - 8), exact.
__device__ inline uint32_t nib2(uint32_t x, int sh)
{
    const half2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    return h2_bits(bits_h2(((x >> sh) & 0x000F000Fu) | 0x64006400u) - off);
}

// One dword of 4 bytes b0..b3 -> low nibbles in order (b0, b2, b1, b3).
__device__ inline void deq_q4_lo(uint32_t x, uint32_t &a, uint32_t &b) { a = nib2(x, 0); b = nib2(x, 8); }
__device__ inline void deq_q4_hi(uint32_t x, uint32_t &a, uint32_t &b) { a = nib2(x, 4); b = nib2(x, 12); }

__device__ inline float half_at(const uint32_t *w, int idx)
{
    uint32_t v = w[idx >> 1];
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((idx & 1) ? (v >> 16) : (v & 0xffffu)));
}

// Channel (within a 32-block) feeding k-slot r of lane group j in the Q.K
// product: it must match how that lane's K codes unpack.
template <int KT>
__device__ inline int qk_chan(int j, int r)
{
    if (KT == KVQ_Q4_0) {
        constexpr int ord[8] = {0, 2, 1, 3, 16, 18, 17, 19};
        return 4 * j + ord[r];
    }
    return 8 * j + r;
}

template <int KT, int VT, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeArgs a)
{
    constexpr int NB = D / 32;   // quant blocks per row
    constexpr int NCT = D / 16;  // 16-channel output tiles
    constexpr int64_t RK = (KT == KVQ_F16) ? 2 * D : (KT == KVQ_Q8_0) ? D : D / 2;
    constexpr int64_t UV = (VT == KVQ_Q4_0) ? D / 2 : D;  // V units per row

    __shared__ float sm_o[WAVES][16][D];
    __shared__ float sm_m[WAVES][16];
    __shared__ float sm_l[WAVES][16];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, j = lane >> 4;
    const int split = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int ctx = a.ctx_len[s];
    const int t_begin = split * a.tps;
    if (t_begin >= ctx)
        return;  // the merge reads only splits that hold tokens
    const int t_end = min(t_begin + a.tps, ctx);
    const int G = a.G;
    const int64_t pair = (int64_t)s * a.Hkv + h;
    const int64_t Tc = a.Tc;

    // Q^T operand: lane (n = head, j) holds 8 channels of each block.
    half8 qb[NB];
    {
        const _Float16 *qrow =
            reinterpret_cast<const _Float16 *>(a.q) + ((int64_t)s * a.Hq + (int64_t)h * G + n) * D;
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int r = 0; r < 8; r++)
                qb[b][r] = (n < G) ? qrow[32 * b + qk_chan<KT>(j, r)] : (_Float16)0.0f;
    }

    const uint8_t *kc = a.kc + pair * Tc * RK;
    const uint16_t *ks = a.ks + pair * Tc * NB;
    const uint8_t *vc = a.vc + pair * (Tc / 8) * UV * 8 * (VT == KVQ_F16 ? 2 : 1);
    const uint16_t *vs = a.vs + pair * (Tc / 8) * NB * 8;
    const float c2 = a.c2;

    float m_run = -INFINITY;  // running max (base-2 units) of head n; equal in all 4 lane groups
    float l_run = 0.0f;       // this lane's share of the running sum
    floatx4 o[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ct++)
        o[ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int tb = t_begin + TILE * wave; tb < t_end; tb += TILE * WAVES) {
        // ---------------- loads
        // K codes, A operand rows: S-tile T, row n -> token tb + 8(n/4) + 4T + n%4
        u32x4 kraw[2][NB];
#pragma unroll
        for (int T = 0; T < 2; T++) {
            const int64_t tok = tb + 8 * (n >> 2) + 4 * T + (n & 3);
            const uint8_t *row = kc + tok * RK;
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (KT == KVQ_F16) {
                    kraw[T][b] = *reinterpret_cast<const u32x4 *>(row + 2 * (32 * b + 8 * j));
                } else if (KT == KVQ_Q8_0) {
                    u32x2 w = *reinterpret_cast<const u32x2 *>(row + 32 * b + 8 * j);
                    kraw[T][b] = u32x4{w.x, w.y, 0u, 0u};
                } else {
                    uint32_t w = *reinterpret_cast<const uint32_t *>(row + 16 * b + 4 * j);
                    kraw[T][b] = u32x4{w, 0u, 0u, 0u};
                }
            }
        }
        // K scales of this lane's 8 output tokens tb+8j .. tb+8j+7, all blocks
        uint32_t ksc[4 * NB];
        if (KT != KVQ_F16) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(ks + (int64_t)(tb + 8 * j) * NB);
#pragma unroll
            for (int i = 0; i < NB; i++) {
                u32x4 w = p[i];
                ksc[4 * i] = w.x, ksc[4 * i + 1] = w.y, ksc[4 * i + 2] = w.z, ksc[4 * i + 3] = w.w;
            }
        }
        // V: group of 8 tokens tb+8j.., unit (channel byte) per output tile
        const int64_t vgrp = (int64_t)(tb >> 3) + j;
        u32x4 vraw[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) {
            if (VT == KVQ_F16) {
                vraw[ct] = *reinterpret_cast<const u32x4 *>(vc + 2 * ((vgrp * UV + 16 * ct + n) * 8));
            } else if (VT == KVQ_Q8_0) {
                u32x2 w = *reinterpret_cast<const u32x2 *>(vc + (vgrp * UV + 16 * ct + n) * 8);
                vraw[ct] = u32x4{w.x, w.y, 0u, 0u};
            } else if ((ct & 1) == 0) {
                u32x2 w = *reinterpret_cast<const u32x2 *>(vc + (vgrp * UV + 16 * (ct >> 1) + n) * 8);
                vraw[ct] = u32x4{w.x, w.y, 0u, 0u};
            } else {
                vraw[ct] = vraw[ct - 1];
            }
        }
        uint32_t vsc[4 * NB];
        if (VT != KVQ_F16) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(vs + (vgrp * NB) * 8);
#pragma unroll
            for (int b = 0; b < NB; b++) {
                u32x4 w = p[b];
                vsc[4 * b] = w.x, vsc[4 * b + 1] = w.y, vsc[4 * b + 2] = w.z, vsc[4 * b + 3] = w.w;
            }
        }

        // ---------------- scores: S^T tile T, lane holds tokens 8j+4T+i, head n
        floatx4 sacc[2];
#pragma unroll
        for (int T = 0; T < 2; T++) {
            sacc[T] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (KT == KVQ_F16) {
                    sacc[T] = mfma(__builtin_bit_cast(half8, kraw[T][b]), qb[b], sacc[T]);
                } else {
                    half8 ka;
                    if (KT == KVQ_Q8_0) {
                        ka = deq_q8(u32x2{kraw[T][b].x, kraw[T][b].y});
                    } else {
                        uint32_t r0, r1, r2, r3;
                        deq_q4_lo(kraw[T][b].x, r0, r1);
                        deq_q4_hi(kraw[T][b].x, r2, r3);
                        ka = pack4(r0, r1, r2, r3);
                    }
                    floatx4 c = mfma(ka, qb[b], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        sacc[T][i] = __builtin_fmaf(half_at(ksc, (4 * T + i) * NB + b), c[i], sacc[T][i]);
                }
            }
        }

        // ---------------- online softmax (base 2), token r = 4T + i of group j
        float x[8];
#pragma unroll
        for (int r = 0; r < 8; r++)
            x[r] = sacc[r >> 2][r & 3] * c2;
        if (tb + TILE > t_end) {
#pragma unroll
            for (int r = 0; r < 8; r++)
                if (tb + 8 * j + r >= t_end)
                    x[r] = -INFINITY;
        }
        float mt = x[0];
#pragma unroll
        for (int r = 1; r < 8; r++)
            mt = fmaxf(mt, x[r]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float p[8];
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; r++) {
            p[r] = __builtin_amdgcn_exp2f(x[r] - m_new);
            psum += p[r];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
            o[ct] *= alpha;

        // ---------------- O^T += V^T . P'
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) {
            const int b = ct >> 1;
            half8 va, pb;
            if (VT == KVQ_F16) {
                va = __builtin_bit_cast(half8, vraw[ct]);
#pragma unroll
                for (int r = 0; r < 8; r++)
                    pb[r] = (_Float16)p[r];
            } else if (VT == KVQ_Q8_0) {
                va = deq_q8(u32x2{vraw[ct].x, vraw[ct].y});
#pragma unroll
                for (int r = 0; r < 8; r++)
                    pb[r] = (_Float16)(p[r] * half_at(vsc, 8 * b + r));
            } else {
                uint32_t r0, r1, r2, r3;
                if ((ct & 1) == 0) {
                    deq_q4_lo(vraw[ct].x, r0, r1);
                    deq_q4_lo(vraw[ct].y, r2, r3);
                } else {
                    deq_q4_hi(vraw[ct].x, r0, r1);
                    deq_q4_hi(vraw[ct].y, r2, r3);
                }
                va = pack4(r0, r1, r2, r3);  // token order 0,2,1,3,4,6,5,7
                constexpr int ord[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
                for (int r = 0; r < 8; r++)
                    pb[r] = (_Float16)(p[ord[r]] * half_at(vsc, 8 * b + ord[r]));
            }
            o[ct] = mfma(va, pb, o[ct]);
        }
    }

    // ---------------- wave totals, then merge the four waves in LDS
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (n < G) {
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                sm_o[wave][n][16 * ct + 4 * j + i] = o[ct][i];
        if (j == 0) {
            sm_m[wave][n] = m_run;
            sm_l[wave][n] = l_tot;
        }
    }
    __syncthreads();

    const int Dp = D + 2;
    float *ws = a.ws + ((((int64_t)s * a.Hq + (int64_t)h * G) * a.n_splits) + split) * Dp;
    const int64_t head_stride = (int64_t)a.n_splits * Dp;
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int g = idx / D, c = idx - g * D;
        float M = sm_m[0][g];
#pragma unroll
        for (int w = 1; w < WAVES; w++)
            M = fmaxf(M, sm_m[w][g]);
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; w++) {
            const float e = (sm_m[w][g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sm_m[w][g] - M);
            acc += sm_o[w][g][c] * e;
            lsum += sm_l[w][g] * e;
        }
        float *dst = ws + g * head_stride;
        dst[c] = acc;
        if (c == 0) {
            dst[D] = M;
            dst[D + 1] = lsum;
        }
    }
}

// out = sum_j O_j 2^(m_j - M) / sum_j l_j 2^(m_j - M) over the splits that
// hold tokens.  One workgroup per (query head, sequence), one lane per channel.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const MergeArgs a)
{
    const int hq = blockIdx.x, s = blockIdx.y, c = threadIdx.x;
    const int ctx = a.ctx_len[s];
    const int nsp = (ctx + a.tps - 1) / a.tps;
    const int Dp = D + 2;
    const float *base = a.ws + (((int64_t)s * a.Hq + hq) * a.n_splits) * Dp;
    float M = -INFINITY;
    for (int sp = 0; sp < nsp; sp++)
        M = fmaxf(M, base[sp * Dp + D]);
    float acc = 0.0f, l = 0.0f;
    for (int sp = 0; sp < nsp; sp++) {
        const float e = __builtin_amdgcn_exp2f(base[sp * Dp + D] - M);
        acc += base[sp * Dp + c] * e;
        l += base[sp * Dp + D + 1] * e;
    }
    a.out[((int64_t)s * a.Hq + hq) * D + c] = acc / l;
}

template <int KT, int VT, int D>
hipError_t launch_dec(const DecodeArgs &a, int n_seqs, hipStream_t st)
{
    dim3 grid(a.n_splits, a.Hkv, n_seqs);
    hipLaunchKernelGGL((decode_split_kernel<KT, VT, D>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dec_d(int kt, int vt, const DecodeArgs &a, int n_seqs, hipStream_t st)
{
#define KVQ_D(K, V) \
    if (kt == K && vt == V) return launch_dec<K, V, D>(a, n_seqs, st);
    KVQ_D(KVQ_F16, KVQ_F16) KVQ_D(KVQ_F16, KVQ_Q8_0) KVQ_D(KVQ_F16, KVQ_Q4_0)
    KVQ_D(KVQ_Q8_0, KVQ_F16) KVQ_D(KVQ_Q8_0, KVQ_Q8_0) KVQ_D(KVQ_Q8_0, KVQ_Q4_0)
    KVQ_D(KVQ_Q4_0, KVQ_F16) KVQ_D(KVQ_Q4_0, KVQ_Q8_0) KVQ_D(KVQ_Q4_0, KVQ_Q4_0)
#undef KVQ_D
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(int kt, int vt, int D, const DecodeArgs &a, int n_seqs, hipStream_t st)
{
    switch (D) {
    case 64: return launch_dec_d<64>(kt, vt, a, n_seqs, st);
    case 128: return launch_dec_d<128>(kt, vt, a, n_seqs, st);
    case 256: return launch_dec_d<256>(kt, vt, a, n_seqs, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_merge(int D, const MergeArgs &a, int n_seqs, hipStream_t st)
{
    dim3 grid(a.Hq, n_seqs);
    switch (D) {
    case 64: hipLaunchKernelGGL((decode_merge_kernel<64>), grid, dim3(64), 0, st, a); break;
    case 128: hipLaunchKernelGGL((decode_merge_kernel<128>), grid, dim3(128), 0, st, a); break;
    case 256: hipLaunchKernelGGL((decode_merge_kernel<256>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
