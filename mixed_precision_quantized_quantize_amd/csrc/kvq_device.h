// kvq_device.h -- device-side building blocks shared by the decode and the
// prefill kernels: binary16 operand unpacking of the block formats, the
// 32-token tile geometry in LDS with its bank swizzles, and the
// direct-to-LDS tile copy.  Internal; not part of the C ABI.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace dev {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
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

// (y & mask) | (c & ~mask) in one instruction.
__device__ inline uint32_t bfi(uint32_t mask, uint32_t y, uint32_t c)
{
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(y), "v"(c));
    return r;
}

// 8 int8 codes -> 8 exact binary16 values: bias to unsigned, place each byte
// under the exponent pattern 0x64 (binary16 1024 + u), subtract 1152.
__device__ inline half8 deq_q8(uint32_t w0, uint32_t w1)
{
    const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
    const half2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    uint32_t r0 = h2_bits(bits_h2(__builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u)) - off);
    uint32_t r1 = h2_bits(bits_h2(__builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u)) - off);
    uint32_t r2 = h2_bits(bits_h2(__builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u)) - off);
    uint32_t r3 = h2_bits(bits_h2(__builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)) - off);
    return pack4(r0, r1, r2, r3);
}

// Two q4_0 code bytes in the low bytes of each 16-bit half of y -> binary16
// pairs (c - 8) of their low nibbles and of their high nibbles, exact:
// low:  binary16 1024 + c       minus 1032
// high: binary16 1024 + 16 c    times 1/16 minus 72
__device__ inline void deq_q4_pair(uint32_t y, uint32_t &lo, uint32_t &hi)
{
    const uint32_t e = 0x64006400u;
    const half2 k1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2 k72 = {(_Float16)-72.0f, (_Float16)-72.0f};
    lo = h2_bits(bits_h2(bfi(0x000F000Fu, y, e)) - k1032);
    hi = h2_bits(__builtin_elementwise_fma(bits_h2(bfi(0x00F000F0u, y, e)), k16, k72));
}

// max over the four lanes n, n+16, n+32, n+48 (the lane groups of one score
// row) with two lane swaps, no LDS round trip.
__device__ inline float max_lane_groups(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // {lanes 0-31 twice}, {32-63 twice}
    const float m = __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    const uint32_t w = __builtin_bit_cast(uint32_t, m);
    const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);  // rows {0,0,2,2}, {1,1,3,3}
    return __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}

// NaN-propagating maximum (v_maximum3_f32): fmaxf would first canonicalize
// every MFMA result with an extra v_max_f32.  Scores are finite, or -inf
// where masked (a masked key's garbage score is replaced before).
__device__ inline float max3(float a, float b, float c)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// q5_0 codes (c = nibble + 16 * fifth bit) -> binary16 (c - 16), exact: the
// nibble goes to bits 4..7 and the fifth bit to bit 8 of a binary16 half
// under the exponent pattern 0x6400 (binary16 1024 + 16 c), then times 1/16
// minus 80.  q5_pair builds two such values from the bytes of two words: nib
// holds the nibbles at bits 4..7 of its bytes, fifth the fifth bits at bit
// 0 of its bytes (the other bits of both are ignored); sel picks bytes
// (0, 1) or (2, 3) of each.
__device__ inline uint32_t q5_pair(uint32_t fifth, uint32_t nib, uint32_t sel)
{
    const half2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2 k80 = {(_Float16)-80.0f, (_Float16)-80.0f};
    const uint32_t y = __builtin_amdgcn_perm(fifth, nib, sel);  // half k: nib byte, fifth byte
    return h2_bits(__builtin_elementwise_fma(bits_h2(bfi(0x01F001F0u, y, 0x64006400u)), k16, k80));
}
constexpr uint32_t Q5_SEL01 = 0x05010400u, Q5_SEL23 = 0x07030602u;

// Bit k of a 4-bit value -> bit 0 of byte k (the partial products of the
// 24-bit multiply occupy disjoint bit ranges, so nothing carries).
__device__ inline uint32_t spread4(uint32_t v4) { return __umul24(v4, 0x00204081u); }

// q5_0 K codes of one block for one lane: w = code bytes 4j..4j+3 of the
// token's row (elements 4j+k low, 16+4j+k high), x = the block's high-bit
// word, sh = 4j (bits sh..sh+3: fifth bits of elements 4j..4j+3, bits
// 16+sh..: of elements 16+4j..).
__device__ inline half8 k_operand_q5(uint32_t w, uint32_t x, int sh)
{
    const uint32_t fl = spread4(__builtin_amdgcn_ubfe(x, sh, 4));
    const uint32_t fh = spread4(__builtin_amdgcn_ubfe(x, 16 + sh, 4));
    const uint32_t wl = w << 4;  // low nibbles to bits 4..7
    return pack4(q5_pair(fl, wl, Q5_SEL01), q5_pair(fl, wl, Q5_SEL23), q5_pair(fh, w, Q5_SEL01),
                 q5_pair(fh, w, Q5_SEL23));
}

// q5_0 V operand of one block: the lane's code byte n (element n low, n+16
// high) for tokens 0..7 in w (bytes of tokens 0..3 in w.x, 4..7 in w.y) and
// those tokens' high-bit words h[0..7] -> the two operands (channel tiles
// of elements n and n+16), binary16 (code - 16).  Per four tokens, byte
// permutes gather the byte of each word that holds element n's fifth bit
// (byte n/8) and the one with element n+16's (byte 2 + n/8); a rotation
// moves bit n%8 of every byte to bit 0.
__device__ inline void v_operand_q5(u32x2 w, const uint32_t (&h)[8], int n, half8 &va0, half8 &va1)
{
    const uint32_t gsel = (n & 8) ? 0x07030501u : 0x06020400u;  // [a.bn, b.bn, a.b(2+n), b.b(2+n)]
    const uint32_t rot = (uint32_t)(n & 7);
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int q = 0; q < 2; q++) {  // tokens 4q .. 4q+3
        const uint32_t wq = q ? w.y : w.x;
        const uint32_t p01 = __builtin_amdgcn_perm(h[4 * q + 1], h[4 * q], gsel);
        const uint32_t p23 = __builtin_amdgcn_perm(h[4 * q + 3], h[4 * q + 2], gsel);
        const uint32_t t0 = __builtin_amdgcn_perm(p23, p01, 0x05040100u);  // byte i: token 4q+i, element n
        const uint32_t t1 = __builtin_amdgcn_perm(p23, p01, 0x07060302u);  // element n+16
        const uint32_t f0 = __builtin_amdgcn_alignbit(t0, t0, rot), f1 = __builtin_amdgcn_alignbit(t1, t1, rot);
        const uint32_t wl = wq << 4;
        lo[2 * q] = q5_pair(f0, wl, Q5_SEL01);
        lo[2 * q + 1] = q5_pair(f0, wl, Q5_SEL23);
        hi[2 * q] = q5_pair(f1, wq, Q5_SEL01);
        hi[2 * q + 1] = q5_pair(f1, wq, Q5_SEL23);
    }
    va0 = pack4(lo[0], lo[1], lo[2], lo[3]);
    va1 = pack4(hi[0], hi[1], hi[2], hi[3]);
}

// turbo3 codebook: the 8 Lloyd-Max levels of N(0,1) in binary16 (-2.152,
// -1.344, -0.756, -0.2451, 0.2451, 0.756, 1.344, 2.152), two per word with
// the even entry in the low half.
constexpr uint32_t TQ3_L01 = 0xBD60C04Eu, TQ3_L23 = 0xB3D8BA0Cu, TQ3_L45 = 0x3A0C33D8u, TQ3_L67 = 0x404E3D60u;

// The same table split by byte: byte e of TQ3_LO03/TQ3_LO47 is the low byte
// of entry e / e+4, and likewise TQ3_HI* for the high bytes -- so that one
// byte permute looks up four entries at once.
constexpr uint32_t tq3_bytes(uint32_t a, uint32_t b, int sh)
{
    return ((a >> sh) & 0xFFu) | ((a >> (16 + sh)) & 0xFFu) << 8 | ((b >> sh) & 0xFFu) << 16 |
           ((b >> (16 + sh)) & 0xFFu) << 24;
}
constexpr uint32_t TQ3_LO03 = tq3_bytes(TQ3_L01, TQ3_L23, 0), TQ3_LO47 = tq3_bytes(TQ3_L45, TQ3_L67, 0);
constexpr uint32_t TQ3_HI03 = tq3_bytes(TQ3_L01, TQ3_L23, 8), TQ3_HI47 = tq3_bytes(TQ3_L45, TQ3_L67, 8);
static_assert(TQ3_LO03 == 0xD80C604Eu && TQ3_HI47 == 0x403D3A33u, "byte tables of the codebook");

// Four levels at once: byte i of c is the 3-bit code of value i; the result
// is values 0, 1 (lo01) and 2, 3 (lo23) as binary16 pairs, value 0 / 2 in the
// low half.
__device__ inline void tq3_quad(uint32_t c, uint32_t &p01, uint32_t &p23)
{
    const uint32_t lo = __builtin_amdgcn_perm(TQ3_LO47, TQ3_LO03, c);  // low bytes of the four levels
    const uint32_t hi = __builtin_amdgcn_perm(TQ3_HI47, TQ3_HI03, c);  // their high bytes
    p01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    p23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// turbo3 V operand of one block: the lane's code byte n&7 for tokens 0..7
// in w (2-bit codes of elements n&7, +8, +16, +24 at bits 0, 2, 4, 6; tokens
// 0..3 in w.x, 4..7 in w.y) and the tokens' third-bit words h[0..7] -> the
// two operands (channel tiles of elements n and n+16) as binary16 levels.
// Per four tokens, byte permutes gather the byte of each word that holds
// element n's third bit (byte n/8) and the one with element n+16's (byte
// 2 + n/8) into one word each; a rotation moves bit n%8 of every byte to bit
// 2, beside the 2-bit codes, and the resulting 3-bit codes select the
// levels' bytes.
__device__ inline void v_operand_tq3(u32x2 w, const uint32_t (&h)[8], int n, half8 &va0, half8 &va1)
{
    const int sh0 = 2 * (n >> 3), sh1 = sh0 + 4;                  // bit offsets of elements n and n+16
    const uint32_t gsel = (n & 8) ? 0x07030501u : 0x06020400u;      // [a.bn, b.bn, a.b(2+n), b.b(2+n)]
    const uint32_t rot = (uint32_t)((n & 7) - 2) & 31u;             // rotate right: bit n%8 -> bit 2
    uint32_t r0[4], r1[4];
#pragma unroll
    for (int q = 0; q < 2; q++) {  // tokens 4q .. 4q+3
        const uint32_t wq = q ? w.y : w.x;
        const uint32_t p01 = __builtin_amdgcn_perm(h[4 * q + 1], h[4 * q], gsel);
        const uint32_t p23 = __builtin_amdgcn_perm(h[4 * q + 3], h[4 * q + 2], gsel);
        const uint32_t t0 = __builtin_amdgcn_perm(p23, p01, 0x05040100u);  // byte i: token 4q+i, element n
        const uint32_t t1 = __builtin_amdgcn_perm(p23, p01, 0x07060302u);  // element n+16
        const uint32_t c0 = bfi(0x04040404u, __builtin_amdgcn_alignbit(t0, t0, rot), (wq >> sh0) & 0x03030303u);
        const uint32_t c1 = bfi(0x04040404u, __builtin_amdgcn_alignbit(t1, t1, rot), (wq >> sh1) & 0x03030303u);
        tq3_quad(c0, r0[2 * q], r0[2 * q + 1]);
        tq3_quad(c1, r1[2 * q], r1[2 * q + 1]);
    }
    va0 = pack4(r0[0], r0[1], r0[2], r0[3]);
    va1 = pack4(r1[0], r1[1], r1[2], r1[3]);
}

// turbo3's rotation signs: element i of a block is negated where bit i is set.
constexpr uint32_t TQ3_SIGNS = 0x9E3779B9u;

// K codes of one block for one lane -> A operand (8 channels of one token).
template <int KT>
__device__ inline half8 k_operand(const uint32_t *w)
{
    if (KT == KVQ_F16)
        return pack4(w[0], w[1], w[2], w[3]);
    if (KT == KVQ_Q8_0)
        return deq_q8(w[0], w[1]);
    // q4_0: bytes 4j..4j+3 hold elements 4j+k (low) and 16+4j+k (high)
    uint32_t l01, h01, l23, h23;
    deq_q4_pair(__builtin_amdgcn_perm(w[0], w[0], 0x0C010C00u), l01, h01);
    deq_q4_pair(__builtin_amdgcn_perm(w[0], w[0], 0x0C030C02u), l23, h23);
    return pack4(l01, l23, h01, h23);
}

// Channel (within a 32-block) carried by k-slot r of lane group j in the Q.K
// product; it must match how k_operand unpacks that lane's codes.
template <int KT>
__device__ inline int qk_chan(int j, int r)
{
    if (KT == KVQ_Q4_0 || KT == KVQ_Q5_0)
        return (r < 4) ? 4 * j + r : 16 + 4 * j + (r - 4);
    return 8 * j + r;
}

// ------------------------------------------------------------------ tile geometry
// One wave stages one 32-token tile in LDS: K codes (token-major rows), K
// scales, K high bits (q5_0), V codes (8-token groups), V scales, V high bits
// (q5_0) -- contiguous ranges of the planes, copied with direct-to-LDS
// 16-byte loads (every instruction reads one contiguous kilobyte) and 4-byte
// loads for the small ranges.  16-byte chunks are XOR-swizzled within a K row / V
// group so that the MFMA-operand reads below hit distinct LDS banks.
template <int KT, int VT, int D>
struct Geo {
    static constexpr int NB = D / 32, NCT = D / 16;
    static constexpr int RK = row_code_bytes(KT, D);  // K row code bytes
    static constexpr int RV = row_code_bytes(VT, D);  // V row code bytes
    static constexpr int K_BYTES = TILE * RK;
    static constexpr int KS_BYTES = (KT == KVQ_F16) ? 0 : TILE * NB * 2;
    static constexpr int KH_BYTES = (KT == KVQ_Q5_0) ? TILE * NB * 4 : 0;
    static constexpr int V_BYTES = TILE * RV;
    static constexpr int VS_BYTES = (VT == KVQ_F16) ? 0 : TILE * NB * 2;
    static constexpr int VH_BYTES = has_bit_words(VT) ? TILE * NB * 4 : 0;
    static constexpr int K_OFF = 0, KS_OFF = K_BYTES, KH_OFF = KS_OFF + KS_BYTES, V_OFF = KH_OFF + KH_BYTES;
    static constexpr int VS_OFF = V_OFF + V_BYTES, VH_OFF = VS_OFF + VS_BYTES;
    static constexpr int BYTES = VH_OFF + VH_BYTES;  // one wave's tile
    // copy instructions of one tile: 1 KB each for codes, 256 B each (128 B
    // on half the lanes) for scales and high bits
    // (turbo3 V at head_dim 64 is half a kilobyte: one instruction on half the lanes)
    static constexpr int NK = K_BYTES / 1024, NV = (V_BYTES + 1023) / 1024;
    static constexpr int NKS = (KT == KVQ_F16) ? 0 : (KS_BYTES == 128 ? 1 : KS_BYTES / 256);
    static constexpr int NVS = (VT == KVQ_F16) ? 0 : (VS_BYTES == 128 ? 1 : VS_BYTES / 256);
    static constexpr int NKH = KH_BYTES / 256, NVH = VH_BYTES / 256;
    static constexpr int NDMA = NK + NKS + NKH + NV + NVS + NVH;
    static constexpr int CPR = RK / 16;              // 16-byte chunks per K row
    static constexpr int CPG = 8 * RV / 16;          // 16-byte chunks per 8-token V group
    static constexpr int LDS_A = WAVES * BYTES;
};

// XOR swizzle of the chunk index within K row r (bank-conflict-free reads of
// the Q.K operand for every type and head_dim; chosen with a bank model).
template <int CPR>
__device__ inline int kswz(int r)
{
    if (CPR <= 4)
        return (r ^ (r >> 3)) & (CPR - 1);
    if (CPR == 8)
        return ((r >> 1) ^ (r >> 2)) & 7;
    return (r ^ (r >> 1)) & (CPR - 1);
}
template <int VT, int CPG>
__device__ inline int vswz(int g)
{
    return (VT == KVQ_F16) ? 0 : (8 * g) & (CPG - 1);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Buffer resource over one plane range [base, base + bytes): word 3 selects
// raw 32-bit data; offsets past `bytes` read as zero instead of faulting.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache policy of a load: CPOL_DEFAULT, or CPOL_STREAM (the "nt" bit) for
// data read once -- a decode call reads each cache byte once, and streaming
// loads measured about 11% more bandwidth than default ones on MI355X.
constexpr int CPOL_DEFAULT = 0, CPOL_STREAM = 2;

// 64 lanes x `size` bytes (lane l from voffset_l + soffset) into LDS at
// dst + l * size; dst and soffset are wave-uniform.
template <int SIZE, int CPOL = CPOL_DEFAULT>
__device__ inline void dma(__amdgpu_buffer_rsrc_t r, int voffset, int soffset, void *dst)
{
    static_assert(SIZE == 16 || SIZE == 4, "lane placement checked for 4- and 16-byte copies only");
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, voffset, soffset, 0, CPOL);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 4, voffset, soffset, 0, CPOL);
}

// Per-lane constant byte offsets of the tile copy (source side, relative to
// the tile's first K row / first V group).
template <int KT, int VT, int D>
struct DmaOffsets {
    using g = Geo<KT, VT, D>;
    int k[g::K_BYTES / 1024];
    int v[g::NV];
    __device__ void init(int lane)
    {
#pragma unroll
        for (int i = 0; i < g::K_BYTES / 1024; i++) {
            const int sl = 64 * i + lane, r = sl / g::CPR, c = (sl % g::CPR) ^ kswz<g::CPR>(r);
            k[i] = r * g::RK + 16 * c;
        }
#pragma unroll
        for (int i = 0; i < g::NV; i++) {
            const int sl = 64 * i + lane, grp = sl / g::CPG, c = (sl % g::CPG) ^ vswz<VT, g::CPG>(grp);
            v[i] = grp * (8 * g::RV) + 16 * c;
        }
    }
};

// Resources over this (sequence, kv head)'s K and V ranges.
struct PairRsrc {
    __amdgpu_buffer_rsrc_t kc, ks, kh, vc, vs, vh;
};

// Copies one tile; with nparts > 1 the copy instructions are dealt out
// round-robin and this caller issues only those of index % nparts == part
// (waves of one workgroup sharing a tile).  CPOL: cache policy of the loads.
template <int KT, int VT, int D, int CPOL = CPOL_DEFAULT>
__device__ inline void issue_tile(uint8_t *buf, int tb, int lane, const DmaOffsets<KT, VT, D> &off, const PairRsrc &r,
                                  int part = 0, int nparts = 1)
{
    using g = Geo<KT, VT, D>;
    // instruction index: K codes, K scales, K high bits, V codes, V scales,
    // V high bits
    constexpr int I_KS = g::NK, I_KH = I_KS + g::NKS, I_V = I_KH + g::NKH, I_VS = I_V + g::NV;
    constexpr int I_VH = I_VS + g::NVS;
    const int kbase = tb * g::RK;
#pragma unroll
    for (int i = 0; i < g::NK; i++)
        if (i % nparts == part)
            dma<16, CPOL>(r.kc, off.k[i], kbase, buf + g::K_OFF + 1024 * i);
    if (KT != KVQ_F16) {
        const int sbase = tb * g::NB * 2;
        if (g::KS_BYTES == 128) {
            if (I_KS % nparts == part && lane < 32)  // 4 bytes on half the lanes (lane l lands at +4 l)
                dma<4, CPOL>(r.ks, 4 * lane, sbase, buf + g::KS_OFF);
        } else {
#pragma unroll
            for (int i = 0; i < g::NKS; i++)
                if ((I_KS + i) % nparts == part)
                    dma<4, CPOL>(r.ks, 256 * i + 4 * lane, sbase, buf + g::KS_OFF + 256 * i);
        }
    }
    if (KT == KVQ_Q5_0) {  // one word per (token, block), token-major
        const int hbase = tb * g::NB * 4;
#pragma unroll
        for (int i = 0; i < g::NKH; i++)
            if ((I_KH + i) % nparts == part)
                dma<4, CPOL>(r.kh, 256 * i + 4 * lane, hbase, buf + g::KH_OFF + 256 * i);
    }
    const int vbase = (tb >> 3) * 8 * g::RV;
#pragma unroll
    for (int i = 0; i < g::NV; i++)
        if ((I_V + i) % nparts == part && (g::V_BYTES % 1024 == 0 || 1024 * i + 16 * lane < g::V_BYTES))
            dma<16, CPOL>(r.vc, off.v[i], vbase, buf + g::V_OFF + 1024 * i);
    if (VT != KVQ_F16) {
        const int sbase = (tb >> 3) * g::NB * 16;
        if (g::VS_BYTES == 128) {
            if (I_VS % nparts == part && lane < 32)
                dma<4, CPOL>(r.vs, 4 * lane, sbase, buf + g::VS_OFF);
        } else {
#pragma unroll
            for (int i = 0; i < g::NVS; i++)
                if ((I_VS + i) % nparts == part)
                    dma<4, CPOL>(r.vs, 256 * i + 4 * lane, sbase, buf + g::VS_OFF + 256 * i);
        }
    }
    if (has_bit_words(VT)) {  // one word per (token, block), 8-token groups
        const int hbase = (tb >> 3) * g::NB * 32;
#pragma unroll
        for (int i = 0; i < g::NVH; i++)
            if ((I_VH + i) % nparts == part)
                dma<4, CPOL>(r.vh, 256 * i + 4 * lane, hbase, buf + g::VH_OFF + 256 * i);
    }
}

// turbo3 values: rotate an output accumulated in the rotated basis back,
// x = s.(H y)/32 per 32-channel block, for a lane's rows in the matrix-core
// output layout: o[ct][i] holds channel 16 ct + 4 j + i (j = lane / 16) of
// the lane's row.  Channel 32 b + e sits at e = 16 (ct - 2 b) + 4 j + i:
// butterflies of span 1, 2 over i, 4, 8 over the lane groups j (lanes 16
// and 32 apart), 16 over the parity of ct; then the signs and 1/32.
template <int NCT>
__device__ inline void rotate_back_tiles(floatx4 (&o)[NCT], const int lane)
{
    const int j = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < NCT; ct++) {
        floatx4 &v = o[ct];
        const float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
        v = floatx4{a0 + a2, a1 + a3, a0 - a2, a1 - a3};
#pragma unroll
        for (int lm = 16; lm <= 32; lm <<= 1) {
            const bool upper = (lane & lm) != 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float other = __shfl_xor(v[i], lm);
                v[i] = upper ? other - v[i] : v[i] + other;
            }
        }
    }
#pragma unroll
    for (int b = 0; b < NCT / 2; b++) {
        const floatx4 lo = o[2 * b], hi = o[2 * b + 1];
        o[2 * b] = lo + hi;
        o[2 * b + 1] = lo - hi;
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ct++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = 16 * (ct & 1) + 4 * j + i;
            o[ct][i] *= ((TQ3_SIGNS >> e) & 1u) ? -0.03125f : 0.03125f;
        }
}

__device__ inline float half_at(const uint32_t *w, int idx)
{
    uint32_t v = w[idx >> 1];
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((idx & 1) ? (v >> 16) : (v & 0xffffu)));
}


}  // namespace dev
}  // namespace kvq
