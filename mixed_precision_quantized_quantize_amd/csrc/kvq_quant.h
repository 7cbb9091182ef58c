// kvq_quant.h -- the block quantizer of one 32-element block, shared by the
// append kernel and the decode kernel's fused one-row append.  Four lanes own
// one block; the block's |x| maximum (q8_0) or signed maximum (q4_0, q5_0) is
// reduced across the four lanes with cross-lane shuffles, then every lane
// writes its own codes.  The arithmetic follows the contract in kvq.h bit for
// bit: binary32 scale, one rounding to binary16, codes against the stored
// scale's binary32 reciprocal, q8_0 rounding half away from zero, q4_0 / q5_0
// product and +8.5 / +16.5 rounded separately (no multiply-add contraction in
// the functions below).  Internal; not part of the C ABI.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace quant {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ inline uint16_t f2h_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Round half away from zero: v - trunc(v) is exact in binary32.
__device__ inline float round_half_away(float v)
{
#pragma clang fp contract(off)
    float t = __builtin_truncf(v);
    return (__builtin_fabsf(v - t) >= 0.5f) ? t + __builtin_copysignf(1.0f, v) : t;
}

// Element indices held by lane q (0..3) of a block: q8_0 / f16 take 8
// consecutive elements, q4_0 / q5_0 take the 4+4 elements that share its 4
// nibble bytes.
template <int T>
__device__ inline int elem_of(int q, int k)
{
    if (T == KVQ_Q4_0 || T == KVQ_Q5_0)
        return (k < 4) ? 4 * q + k : 16 + 4 * q + (k - 4);
    return 8 * q + k;
}

template <int T>
__device__ inline void load8(const uint16_t *blk, int q, uint16_t (&x)[8])
{
    if (T == KVQ_Q4_0 || T == KVQ_Q5_0) {
        u32x2 a = *reinterpret_cast<const u32x2 *>(blk + 4 * q);
        u32x2 b = *reinterpret_cast<const u32x2 *>(blk + 16 + 4 * q);
        uint32_t w[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
        for (int k = 0; k < 8; k++)
            x[k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
    } else {
        u32x4 a = *reinterpret_cast<const u32x4 *>(blk + 8 * q);
        uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 8; k++)
            x[k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
    }
}

// Quantize one block (this lane's 8 elements) and store codes + scale.
// qh: q5_0's high-bit words (one per row and block, indexed like the
// scales), unused for the other types.
template <int T, int ROLE>
__device__ inline void quant_store(const uint16_t *blk, int q, uint8_t *codes, uint16_t *scales, uint32_t *qh,
                                   int64_t pair, int64_t t, int b, int D, int Tc)
{
#pragma clang fp contract(off)
    const int NB = D / 32;
    const int64_t R = row_code_bytes(T, D);
    uint16_t xb[8];
    load8<T>(blk, q, xb);

    // Where unit u of this token lives (units: bytes, or binary16 for f16).
    const int64_t U = (T == KVQ_F16) ? D : R;
    auto unit_index = [&](int64_t u) -> int64_t {
        if (ROLE == 0)
            return (pair * Tc + t) * U + u;
        return ((pair * (Tc / 8) + t / 8) * U + u) * 8 + (t & 7);
    };
    auto scale_index = [&]() -> int64_t {
        if (ROLE == 0)
            return (pair * Tc + t) * NB + b;
        return ((pair * (Tc / 8) + t / 8) * NB + b) * 8 + (t & 7);
    };

    if (T == KVQ_F16) {
        uint16_t *dst = reinterpret_cast<uint16_t *>(codes);
        if (ROLE == 0) {
            u32x4 v;
            v.x = xb[0] | ((uint32_t)xb[1] << 16);
            v.y = xb[2] | ((uint32_t)xb[3] << 16);
            v.z = xb[4] | ((uint32_t)xb[5] << 16);
            v.w = xb[6] | ((uint32_t)xb[7] << 16);
            *reinterpret_cast<u32x4 *>(dst + unit_index(32 * b + 8 * q)) = v;
        } else {
#pragma unroll
            for (int k = 0; k < 8; k++)
                dst[unit_index(32 * b + 8 * q + k)] = xb[k];
        }
        return;
    }

    float x[8];
#pragma unroll
    for (int k = 0; k < 8; k++)
        x[k] = h2f(xb[k]);

    float d;
    uint16_t dbits;
    if (T == KVQ_Q8_0) {
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++)
            amax = fmaxf(amax, __builtin_fabsf(x[k]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        float d32 = __fdiv_rn(amax, 127.0f);
        dbits = f2h_bits(d32);
    } else {
        // key = |x| bits (monotonic for finite binary16) , lowest index, sign
        uint32_t key = 0;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            uint32_t e = (uint32_t)elem_of<T>(q, k);
            uint32_t kk = ((uint32_t)(xb[k] & 0x7fff) << 6) | ((31u - e) << 1) | (uint32_t)(xb[k] >> 15);
            key = key > kk ? key : kk;
        }
        uint32_t o = (uint32_t)__shfl_xor((int)key, 1);
        key = key > o ? key : o;
        o = (uint32_t)__shfl_xor((int)key, 2);
        key = key > o ? key : o;
        uint32_t absbits = key >> 6;
        float m = (absbits == 0) ? 0.0f : h2f((uint16_t)(absbits | ((key & 1u) << 15)));
        float d32 = __fdiv_rn(m, (T == KVQ_Q5_0) ? -16.0f : -8.0f);
        dbits = f2h_bits(d32);
    }
    d = h2f(dbits);
    const float id = (d != 0.0f) ? __fdiv_rn(1.0f, d) : 0.0f;

    if (T == KVQ_Q8_0) {
        uint8_t c[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float v = x[k] * id;  // plain binary32 product (contraction is off in this file)
            float r = round_half_away(v);
            r = fminf(127.0f, fmaxf(-127.0f, r));
            c[k] = (uint8_t)(int8_t)(int)r;
        }
        if (ROLE == 0) {
            u32x2 v;
            v.x = c[0] | (c[1] << 8) | (c[2] << 16) | ((uint32_t)c[3] << 24);
            v.y = c[4] | (c[5] << 8) | (c[6] << 16) | ((uint32_t)c[7] << 24);
            *reinterpret_cast<u32x2 *>(codes + unit_index(32 * b + 8 * q)) = v;
        } else {
#pragma unroll
            for (int k = 0; k < 8; k++)
                codes[unit_index(32 * b + 8 * q + k)] = c[k];
        }
    } else {
        constexpr float HALF_RANGE = (T == KVQ_Q5_0) ? 16.5f : 8.5f;
        constexpr int TOP = (T == KVQ_Q5_0) ? 31 : 15;
        int c[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float t = x[k] * id;       // rounded product ...
            const float u = t + HALF_RANGE;  // ... then a separately rounded sum: never one fused op
            int ci = (int)__builtin_truncf(u);
            c[k] = ci < 0 ? 0 : (ci > TOP ? TOP : ci);
        }
        uint8_t by[4];
#pragma unroll
        for (int k = 0; k < 4; k++)
            by[k] = (uint8_t)((c[k] & 15) | ((c[k + 4] & 15) << 4));  // element 4q+k low, 16+4q+k high
        if (T == KVQ_Q5_0) {
            // the block's 32 high bits: this lane's 8, then OR over the quad
            uint32_t h = 0;
#pragma unroll
            for (int k = 0; k < 4; k++)
                h |= ((uint32_t)(c[k] >> 4) << (4 * q + k)) | ((uint32_t)(c[k + 4] >> 4) << (16 + 4 * q + k));
            h |= (uint32_t)__shfl_xor((int)h, 1);
            h |= (uint32_t)__shfl_xor((int)h, 2);
            if (q == 0)
                qh[scale_index()] = h;
        }
        if (ROLE == 0) {
            *reinterpret_cast<uint32_t *>(codes + unit_index(16 * b + 4 * q)) =
                by[0] | (by[1] << 8) | (by[2] << 16) | ((uint32_t)by[3] << 24);
        } else {
#pragma unroll
            for (int k = 0; k < 4; k++)
                codes[unit_index(16 * b + 4 * q + k)] = by[k];
        }
    }
    if (q == 0)
        scales[scale_index()] = dbits;
}

}  // namespace quant
}  // namespace kvq
