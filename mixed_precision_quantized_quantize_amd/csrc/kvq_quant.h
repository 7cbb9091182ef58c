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

// One lane's share of a quantized block: its code units in unit order and
// the block's scale and bit word (the same in all four lanes).  Units are the
// bytes of a row's codes (binary16 values for f16); lane q holds NU units
// starting at NU*q within the block.
struct LaneCodes {
    uint16_t dbits;  // binary16 scale (f16: unused)
    uint32_t bits;   // q5_0 high-bit word / turbo3 third-bit word of the block, else 0
    uint32_t w[4];   // the lane's units, little-endian: f16 8 x 2 B, q8_0 8 B, q4_0 / q5_0 4 B, turbo3 2 B
};
template <int T>
constexpr int lane_units() { return (T == KVQ_Q4_0 || T == KVQ_Q5_0) ? 4 : (T == KVQ_TURBO3 ? 2 : 8); }

// turbo3 (values only): the rotated block y = H (s . x) in binary64 -- exact,
// since every partial sum of binary16 inputs is a multiple of 2^-24 below
// 2^21 -- butterflies within the lane's 8 elements and then across the quad;
// scale from max |y|, codes = the nearest of the 8 binary16 Lloyd-Max levels
// of the scaled value (binary32), as a 2-bit plane byte per element group
// (byte j: elements j, j+8, j+16, j+24) and a third-bit word.  Lane q holds
// elements 8q..8q+7 and returns plane bytes 2q, 2q+1.
__device__ inline LaneCodes quant_lane_tq3(const uint16_t *blk, int q)
{
#pragma clang fp contract(off)
    constexpr uint32_t SIGNS = 0x9E3779B9u;
    // the level midpoints (binary32, exact): between -2.152 -1.344 -0.756
    // -0.2451 0.2451 0.756 1.344 2.152 (binary16 values)
    constexpr float LV[8] = {-2.15234375f, -1.34375f, -0.755859375f, -0.2451171875f,
                             0.2451171875f, 0.755859375f, 1.34375f, 2.15234375f};
    uint16_t xb[8];
    load8<KVQ_F16>(blk, q, xb);
    double y[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const double x = (double)h2f(xb[k]);
        y[k] = ((SIGNS >> (8 * q + k)) & 1u) ? -x : x;
    }
#pragma unroll
    for (int len = 1; len < 8; len <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i += 2 * len)
#pragma unroll
            for (int k = i; k < i + len; k++) {
                const double a0 = y[k], b0 = y[k + len];
                y[k] = a0 + b0;
                y[k + len] = a0 - b0;
            }
#pragma unroll
    for (int lm = 1; lm <= 2; lm <<= 1) {  // spans 8 and 16: lane bits 0 and 1
        const bool upper = (q & lm) != 0;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const double o = __shfl_xor(y[k], lm);
            y[k] = upper ? o - y[k] : y[k] + o;
        }
    }
    double m = 0.0;
#pragma unroll
    for (int k = 0; k < 8; k++)
        m = fmax(m, __builtin_fabs(y[k]));
    m = fmax(m, __shfl_xor(m, 1));
    m = fmax(m, __shfl_xor(m, 2));
    const float d32 = __fdiv_rn((float)m, LV[7]);
    LaneCodes lc;
    lc.dbits = f2h_bits(d32);
    const float d = h2f(lc.dbits);
    const float id = (d != 0.0f) ? __fdiv_rn(1.0f, d) : 0.0f;
    uint32_t plane = 0, third = 0;  // this lane's bits of the 2-bit plane bytes 0..7 (two words), third bits
    uint32_t plane_hi = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const float tv = (float)y[k] * id;
        int c = 0;
#pragma unroll
        for (int jj = 0; jj < 7; jj++)
            c += (tv >= (LV[jj] + LV[jj + 1]) * 0.5f) ? 1 : 0;
        const uint32_t bits = (uint32_t)(c & 3) << (8 * (k & 3) + 2 * q);  // byte k, bits 2q
        if (k < 4)
            plane |= bits;
        else
            plane_hi |= bits;
        third |= (uint32_t)(c >> 2) << (8 * q + k);
    }
    plane |= (uint32_t)__shfl_xor((int)plane, 1);
    plane |= (uint32_t)__shfl_xor((int)plane, 2);
    plane_hi |= (uint32_t)__shfl_xor((int)plane_hi, 1);
    plane_hi |= (uint32_t)__shfl_xor((int)plane_hi, 2);
    third |= (uint32_t)__shfl_xor((int)third, 1);
    third |= (uint32_t)__shfl_xor((int)third, 2);
    lc.bits = third;
    lc.w[0] = (((q < 2) ? plane : plane_hi) >> (16 * (q & 1))) & 0xFFFFu;  // bytes 2q, 2q+1
    lc.w[1] = lc.w[2] = lc.w[3] = 0;
    return lc;
}

template <int T>
__device__ inline LaneCodes quant_lane(const uint16_t *blk, int q)
{
#pragma clang fp contract(off)
    if constexpr (T == KVQ_TURBO3)
        return quant_lane_tq3(blk, q);
    LaneCodes lc;
    lc.dbits = 0;
    lc.bits = 0;
    uint16_t xb[8];
    load8<T>(blk, q, xb);
    if (T == KVQ_F16) {
#pragma unroll
        for (int i = 0; i < 4; i++)
            lc.w[i] = xb[2 * i] | ((uint32_t)xb[2 * i + 1] << 16);
        return lc;
    }

    float x[8];
#pragma unroll
    for (int k = 0; k < 8; k++)
        x[k] = h2f(xb[k]);

    if (T == KVQ_Q8_0) {
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++)
            amax = fmaxf(amax, __builtin_fabsf(x[k]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        float d32 = __fdiv_rn(amax, 127.0f);
        lc.dbits = f2h_bits(d32);
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
        lc.dbits = f2h_bits(d32);
    }
    const float d = h2f(lc.dbits);
    const float id = (d != 0.0f) ? __fdiv_rn(1.0f, d) : 0.0f;

    if (T == KVQ_Q8_0) {
        uint32_t c[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float v = x[k] * id;  // plain binary32 product (contraction is off in this file)
            float r = round_half_away(v);
            r = fminf(127.0f, fmaxf(-127.0f, r));
            c[k] = (uint32_t)(uint8_t)(int8_t)(int)r;
        }
        lc.w[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        lc.w[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        lc.w[2] = lc.w[3] = 0;
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
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; k++)  // byte k: element 4q+k low, 16+4q+k high
            w |= (uint32_t)((c[k] & 15) | ((c[k + 4] & 15) << 4)) << (8 * k);
        lc.w[0] = w;
        lc.w[1] = lc.w[2] = lc.w[3] = 0;
        if (T == KVQ_Q5_0) {
            // the block's 32 high bits: this lane's 8, then OR over the quad
            uint32_t h = 0;
#pragma unroll
            for (int k = 0; k < 4; k++)
                h |= ((uint32_t)(c[k] >> 4) << (4 * q + k)) | ((uint32_t)(c[k + 4] >> 4) << (16 + 4 * q + k));
            h |= (uint32_t)__shfl_xor((int)h, 1);
            h |= (uint32_t)__shfl_xor((int)h, 2);
            lc.bits = h;
        }
    }
    return lc;
}

// Quantize one block (this lane's 8 elements) and store codes, scale and bit
// word straight into a plane, for token t of pair `pair`.  ROLE 0: the
// token-major K plane (a lane's units are contiguous: one store); ROLE 1: the
// 8-token interleaved V plane (one store per unit, 8 tokens apart -- the
// bulk append stages whole 8-token groups instead).  qh: the bit words (q5_0,
// turbo3), unused for the other types.
template <int T, int ROLE>
__device__ inline void quant_store(const uint16_t *blk, int q, uint8_t *codes, uint16_t *scales, uint32_t *qh,
                                   int64_t pair, int64_t t, int b, int D, int Tc)
{
    constexpr int NU = lane_units<T>();
    constexpr int W = (T == KVQ_F16) ? 2 : 1;  // bytes per unit
    const int NB = D / 32;
    const int64_t U = row_code_bytes(T, D) / W;  // units per row
    const int64_t UB = U / NB;                    // units per block
    const LaneCodes lc = quant_lane<T>(blk, q);
    const int64_t u0 = UB * b + NU * q;  // the lane's first unit in the row
    const int64_t si = (ROLE == 0) ? (pair * Tc + t) * NB + b : ((pair * (Tc / 8) + t / 8) * NB + b) * 8 + (t & 7);
    if (ROLE == 0) {
        uint8_t *dst = codes + ((pair * Tc + t) * U + u0) * W;
        if (NU * W == 16)
            *reinterpret_cast<u32x4 *>(dst) = u32x4{lc.w[0], lc.w[1], lc.w[2], lc.w[3]};
        else if (NU * W == 8)
            *reinterpret_cast<u32x2 *>(dst) = u32x2{lc.w[0], lc.w[1]};
        else if (NU * W == 4)
            *reinterpret_cast<uint32_t *>(dst) = lc.w[0];
        else
            *reinterpret_cast<uint16_t *>(dst) = (uint16_t)lc.w[0];
    } else {
        const int64_t gbase = (pair * (Tc / 8) + t / 8) * U;
#pragma unroll
        for (int k = 0; k < NU; k++) {
            const int64_t idx = ((gbase + u0 + k) * 8 + (t & 7)) * W;
            if (W == 2)
                *reinterpret_cast<uint16_t *>(codes + idx) = (uint16_t)(lc.w[k >> 1] >> (16 * (k & 1)));
            else
                codes[idx] = (uint8_t)(lc.w[k >> 2] >> (8 * (k & 3)));
        }
    }
    if (q == 0 && T != KVQ_F16) {
        scales[si] = lc.dbits;
        if (T == KVQ_Q5_0 || T == KVQ_TURBO3)
            qh[si] = lc.bits;
    }
}

}  // namespace quant
}  // namespace kvq
