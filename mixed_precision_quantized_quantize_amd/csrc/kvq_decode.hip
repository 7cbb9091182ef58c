// kvq_decode.hip -- flash decode over the quantized cache: one launch per
// call, a persistent streaming kernel whose workgroups also merge their
// partial results.
//
// Flash attention in the sense of the llama.cpp guide's "Flash Attention"
// section (tiled, the score matrix never materialized, exactly softmax
// attention), reading the quantized blocks directly -- the KVSplit page's
// discussion expects the gain "integrated directly into FlashAttention", and
// the llama.cpp issue shows a quantized V cache is only usable that way.
//
// Work split.  Every (sequence, kv head) pair gets k waves (k per sequence)
// in kw = ceil(k/4) workgroups of four waves; wave r = 4*rw + w of the pair
// (workgroup rw, wave w) takes the pair's 32-token tiles r, r+k, r+2k, ...
// so that the k waves stream neighbouring tiles at any moment (a wave with
// r >= k has none).  A wave keeps the copies of its next tiles in flight
// while it computes the current one.
//
// Per tile a wave serves the whole GQA group (up to 16 query heads) of its kv
// head with two matrix-core contractions, both v_mfma_f32_16x16x32_f16:
//   S^T[token][head] = K[token][c] . Q^T[c][head]  -- one MFMA per 16 tokens
//       and 32-channel block; the raw codes are exact in binary16 and the
//       block's K scale multiplies the MFMA result per token;
//   O^T[chan][head] += V^T[chan][token] . P'[token][head]  -- one MFMA per 16
//       channels and 32 tokens; P' = binary16(p) * V scale of (token, block).
// q8_0 and q4_0 codes (both products) and q5_0 keys enter as binary16
// subnormals (a mask or byte permute of the stored bits, no per-element
// arithmetic; q5_0's fifth bits through a second score MFMA); their offset
// comes off per block, through the score MFMA's accumulator input for keys
// and one more MFMA against a constant operand for values.
// The score layout of the first product is exactly the operand layout of the
// second, so probabilities never leave registers.  The V plane stores 8
// tokens interleaved, so a lane's P.V operand (8 tokens of one channel) is
// one 8- or 16-byte load.  Online softmax runs in base 2 (scores times
// scale*log2 e).
//
// Merge.  The four waves of a workgroup combine their (max, sum, output)
// partials in LDS.  A pair served by one workgroup writes its output right
// there.  Otherwise each workgroup writes its combined partial into its slot
// of the workspace and counts itself in on the pair's counter; the workgroup
// that arrives last combines the pair's slots (log-sum-exp, in slot order,
// so that results do not depend on arrival order), writes the output and
// puts the counter back to zero.  The eight XCDs' L2 caches are not coherent
// with each other, and a release fence would write back a whole L2 in every
// workgroup; instead the slots are written and read with device-coherent
// (sc1) stores and loads -- the way the compiler implements relaxed
// agent-scope atomics, which need no L2 writeback -- and a workgroup's slot
// stores have completed (s_waitcnt vmcnt(0)) before its counter increment is
// issued.  No workgroup ever waits for another.
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

using namespace dev;

#ifndef KVQ_DECODE_NBUF
#define KVQ_DECODE_NBUF 2
#endif

// Tile buffers per wave: up to KVQ_DECODE_NBUF, as many as fit in LDS and
// in the vmcnt counter's range.
template <int KT, int VT, int D>
constexpr int decode_nbuf()
{
    using g = Geo<KT, VT, D>;
    constexpr int NDMA = g::NDMA;
    int n = KVQ_DECODE_NBUF;
    while (n > 1 && (n * g::LDS_A + 64 > 160 * 1024 || (n - 1) * NDMA >= 64))
        n--;
    return n;
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), in order.
template <int N, class F>
__device__ inline __attribute__((always_inline)) void static_for(F &&f)
{
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>());
    }
}

// ---- Subnormal operands (decode).  The matrix core multiplies binary16
// subnormals exactly (checked on gfx950: every product and sum of a
// 16x16x32 MFMA with subnormal inputs on either side within 2^-23 of the
// exact sum), so a code u < 1024 whose bits sit in a half as the bare integer
// is the binary16 value u * 2^-24: no exponent pattern to insert and no
// offset to subtract per element.  The code's offset (+128 for q8_0 once its
// sign bit is flipped, +8 for q4_0) is taken out per block instead -- for
// keys through the score MFMA's accumulator input, for values by one more
// MFMA of the same probabilities against a constant operand -- and the 2^-24
// is folded into the softmax scale (keys) or into the output (values).
constexpr float TWO_M24 = 5.9604644775390625e-08f;  // 2^-24
constexpr float TWO_P24 = 16777216.0f;              // 2^24
constexpr uint32_t SUB_NEG8 = 0x80088008u;           // binary16 pair (-8 * 2^-24, -8 * 2^-24)
constexpr uint32_t SUB_NEG128 = 0x80808080u;         // binary16 pair (-128 * 2^-24, -128 * 2^-24)

// 8 int8 codes c -> binary16 (c + 128) * 2^-24, exact: the sign bit flipped,
// each byte alone in a half.
__device__ inline half8 deq_q8_sub(uint32_t w0, uint32_t w1)
{
    const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
    return pack4(__builtin_amdgcn_perm(0u, x0, 0x0C010C00u), __builtin_amdgcn_perm(0u, x0, 0x0C030C02u),
                 __builtin_amdgcn_perm(0u, x1, 0x0C010C00u), __builtin_amdgcn_perm(0u, x1, 0x0C030C02u));
}

// q4_0 K codes of one block for one lane: w = code bytes 4j..4j+3 of the
// token's row (byte k: element 4j+k in the low nibble, 16+4j+k in the high)
// -> k-slots 0..3 = elements 4j, 4j+2, 4j+1, 4j+3 as c * 2^-24 and k-slots
// 4..7 = elements 16+4j, 16+4j+2, 16+4j+1, 16+4j+3 as 16 c * 2^-24 (the high
// nibble left in place; the query channels of those slots carry q / 16).
__device__ inline half8 k_operand_q4_sub(uint32_t w)
{
    const uint32_t w8 = w >> 8;
    return pack4(w & 0x000F000Fu, w8 & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x00F000F0u);
}

// q4_0 V codes of one block for one lane: code byte n of tokens 0..3 (w.x)
// and 4..7 (w.y) -> the operand of element n (low nibbles, c * 2^-24) and of
// element n+16 (high nibbles, 16 c * 2^-24), tokens in order.
__device__ inline void v_operand_q4_sub(u32x2 w, half8 &va0, half8 &va1)
{
    const uint32_t y01 = __builtin_amdgcn_perm(w.x, w.x, 0x0C010C00u), y23 = __builtin_amdgcn_perm(w.x, w.x, 0x0C030C02u);
    const uint32_t y45 = __builtin_amdgcn_perm(w.y, w.y, 0x0C010C00u), y67 = __builtin_amdgcn_perm(w.y, w.y, 0x0C030C02u);
    va0 = pack4(y01 & 0x000F000Fu, y23 & 0x000F000Fu, y45 & 0x000F000Fu, y67 & 0x000F000Fu);
    va1 = pack4(y01 & 0x00F000F0u, y23 & 0x00F000F0u, y45 & 0x00F000F0u, y67 & 0x00F000F0u);
}

// q5_0 K fifth bits of one block for one lane as a second subnormal operand:
// x = the (token, block) high-bit word (bit e: element e), j = lane group.
// Rotated right by 4j - 4, bits 4j+k and 16+4j+k land at bits 4+k and 20+k,
// so word k keeps them: k-slots 2k, 2k+1 = elements 4j+k, 16+4j+k with value
// 2^(4+k) * 2^-24 where the bit is set.  Their query channels carry
// q * 2^-k, which makes each set bit count 16 (the fifth bit's weight).
__device__ inline half8 k_operand_q5_fifth(uint32_t x, int j)
{
    const uint32_t y = __builtin_amdgcn_alignbit(x, x, (uint32_t)(4 * j - 4) & 31u);
    return pack4(y & 0x00100010u, y & 0x00200020u, y & 0x00400040u, y & 0x00800080u);
}

// Cache policy bit of a device-coherent (agent-scope) access: sc1.
constexpr int CPOL_SC1 = 16;

// turbo3 values: rotate a 32-channel block of the output back, x = s.(H y)/32,
// for a quad of channels c .. c+3 (c a multiple of 4) per lane, eight lanes
// per block: butterflies of span 1 and 2 inside the quad, 4, 8, 16 across
// lanes; then the signs and 1/32.
__device__ inline floatx4 rotate_back_quad(floatx4 v, const int c)
{
    const float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
    v = floatx4{a0 + a2, a1 + a3, a0 - a2, a1 - a3};
#pragma unroll
    for (int span = 4; span < 32; span <<= 1) {
        const bool upper = (c & span) != 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float o = __shfl_xor(v[i], span / 4);
            v[i] = upper ? o - v[i] : v[i] + o;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
        v[i] *= ((TQ3_SIGNS >> ((c + i) & 31)) & 1u) ? -0.03125f : 0.03125f;
    return v;
}

// LDS of the final merge: weights and sums of up to KVQ_MAX_WG_PER_PAIR
// slots x 16 query heads.
constexpr int MERGE_SLOTS = KVQ_MAX_WG_PER_PAIR * KVQ_MAX_GROUP;

template <int KT, int VT, int D>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1))) void decode_kernel(const DecodeArgs a)
{
    using g = Geo<KT, VT, D>;
    constexpr int NB = g::NB, NCT = g::NCT;

    // NBUF tile buffers per wave, as many as fit (up to KVQ_DECODE_NBUF),
    // indexed by compile-time constants only, so that the compiler sees that
    // a read of one does not wait for another
    constexpr int NBUF = decode_nbuf<KT, VT, D>();
    __shared__ __attribute__((aligned(16))) uint8_t lds_t[NBUF][g::LDS_A];
    uint8_t *const lds_a = lds_t[0];
    // the arrival verdict of the counter increment
    __shared__ int mrg_last;
    // The workgroup's own merge reuses lds_a once every wave has left its
    // tile loop (per wave and head m and l, then the running sum of O); the
    // final merge's per-(slot, head) weights and sums reuse it after that.
    static_assert(WAVES * 32 * 4 + KVQ_MAX_GROUP * D * 4 <= g::LDS_A, "workgroup merge fits in lds_a");
    static_assert(2 * MERGE_SLOTS * 4 <= g::LDS_A, "final merge fits in lds_a");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
    const int n = lane & 15, j = lane >> 4;
    const int G = a.G, Hkv = a.Hkv;
    const int64_t Tc = a.Tc;
    const int n_pairs = a.n_seqs * Hkv;

    // This workgroup's pair (s, h) and its index rw among the pair's kw
    // workgroups.  The pairs are interleaved over the grid (workgroup b
    // serves pair b mod pairs when every sequence has kw workgroups per pair),
    // so that every pair gets workgroups from early- and late-dispatched
    // parts of the grid alike; otherwise the sequences' first workgroups are
    // binary searched (dependent scalar loads) and the heads of one sequence
    // are interleaved.  slot0 / slot_step: the workspace slots of the pair's
    // workgroups rw' = 0 .. kw-1 are slot0 + rw' * slot_step.
    const int b = blockIdx.x;
    int s = 0, kw = a.kw_uniform, h, rw, slot0, slot_step;
    if (kw > 0) {
        rw = b / n_pairs;
        const int pg = b - rw * n_pairs;
        s = pg / Hkv;
        h = pg - s * Hkv;
        slot0 = pg;
        slot_step = n_pairs;
    } else {
        int hi = a.n_seqs;  // wg_start[s] <= b < wg_start[hi]
        while (hi - s > 1) {
            const int mid = (s + hi) >> 1;
            if (a.wg_start[mid] <= b)
                s = mid;
            else
                hi = mid;
        }
        kw = (a.wg_start[s + 1] - a.wg_start[s]) / Hkv;
        const int local = b - a.wg_start[s];
        rw = local / Hkv;
        h = local - rw * Hkv;
        slot0 = a.wg_start[s] + h;
        slot_step = Hkv;
    }
    const int k = a.k[s];           // waves per pair
    const int r = 4 * rw + wave;    // this wave among them
    const int ctx = a.ctx_len[s];
    const int nt = (ctx + TILE - 1) / TILE;
    const int n_mine = r < k ? (nt - r + k - 1) / k : 0;  // tiles r, r+k, ... below nt
    const int64_t pair = (int64_t)s * Hkv + h;

    // Fused one-row append: the wave that reads the pair's last tile first
    // quantizes the new row into position ctx-1 (one quad of lanes per
    // 32-element block, K blocks then V blocks, the append kernel's
    // quantizer), and waits until the stores are performed before any copy
    // of that tile is issued.  No other wave reads that tile.
    if (a.knew != nullptr && r == (nt - 1) % k) {
        const int quad = lane >> 2, q = lane & 3;
        if (quad < 2 * NB) {
            const int role = quad >= NB, bb = quad - role * NB;
            const uint16_t *blk = (role ? a.vnew : a.knew) + pair * D + 32 * bb;
            if (role == 0)
                quant::quant_store<KT, 0>(blk, q, const_cast<uint8_t *>(a.kc), const_cast<uint16_t *>(a.ks),
                                          const_cast<uint32_t *>(a.kqh), pair, ctx - 1, bb, D, a.Tc);
            else
                quant::quant_store<VT, 1>(blk, q, const_cast<uint8_t *>(a.vc), const_cast<uint16_t *>(a.vs),
                                          const_cast<uint32_t *>(a.vqh), pair, ctx - 1, bb, D, a.Tc);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    PairRsrc rs;
    rs.kc = make_rsrc(a.kc + pair * Tc * g::RK, Tc * g::RK);
    rs.vc = make_rsrc(a.vc + pair * Tc * g::RV, Tc * g::RV);
    if (KT != KVQ_F16)
        rs.ks = make_rsrc(a.ks + pair * Tc * NB, Tc * NB * 2);
    if (VT != KVQ_F16)
        rs.vs = make_rsrc(a.vs + pair * Tc * NB, Tc * NB * 2);
    if (KT == KVQ_Q5_0)
        rs.kh = make_rsrc(a.kqh + pair * Tc * NB, Tc * NB * 4);
    if (has_bit_words(VT))
        rs.vh = make_rsrc(a.vqh + pair * Tc * NB, Tc * NB * 4);

    // Q^T operand: lane (n = head, j) holds 8 channels of each block (8j..
    // for f16/q8_0; 4j.. and 16+4j.. for q4_0 and q5_0, the q4_0 slots
    // reordered below to match k_operand_q4_sub); buffer loads from the
    // scalar base of the pair's Q rows
    //
    // q8_0, q4_0 and q5_0 keys are subnormal operands (the helpers above):
    // the score MFMA of block b then starts from kofs[b] = -offset * 2^-24 *
    // (sum of head n's query over the block's 32 channels), which removes the
    // codes' offset exactly where the raw sum of the MFMA has it, and the
    // scores come out in units of 2^-24 (folded into c2).  q4_0 and q5_0
    // slots 4..7 hold the high nibbles as 16 c: their query channels are
    // q / 16.  q5_0's fifth bits enter through a second MFMA against qb5.
    constexpr bool KSUB = KT == KVQ_Q8_0 || KT == KVQ_Q4_0 || KT == KVQ_Q5_0;
    constexpr bool K5 = KT == KVQ_Q5_0;
    half8 qb[NB];
    floatx4 kofs[KSUB ? NB : 1];
    half8 qb5[K5 ? NB : 1];
    {
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(reinterpret_cast<const _Float16 *>(a.q) + ((int64_t)s * a.Hq + (int64_t)h * G) * D, G * D * 2);
        constexpr bool KNIB = KT == KVQ_Q4_0 || KT == KVQ_Q5_0;  // nibble-packed K
        const int qoff = 2 * (n * D + (KNIB ? 4 * j : 8 * j));
#pragma unroll
        for (int b = 0; b < NB; b++) {
            qb[b] = half8{};
            if (n < G) {  // lanes past the group keep zeros (their loads are not issued)
                if (KNIB) {
                    const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(rq, qoff + 64 * b, 0, 0);
                    const u32x2 hi2 = __builtin_amdgcn_raw_buffer_load_b64(rq, qoff + 64 * b + 32, 0, 0);
                    qb[b] = pack4(lo.x, lo.y, hi2.x, hi2.y);
                } else {
                    qb[b] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 64 * b, 0, 0));
                }
            }
        }
    }
    const float c2 = KSUB ? a.c2 * TWO_P24 : a.c2;

    DmaOffsets<KT, VT, D> doff;
    doff.init(lane);
    // per-lane LDS read offsets of the operands (constant over tiles)
    int k_rd[2][NB];  // K operand of S-tile T, block b
#pragma unroll
    for (int T = 0; T < 2; T++) {
        const int r = 8 * (n >> 2) + 4 * T + (n & 3);
#pragma unroll
        for (int b = 0; b < NB; b++) {
            int c, within;
            if (KT == KVQ_Q8_0) c = 2 * b + (j >> 1), within = 8 * (j & 1);
            else if (KT == KVQ_Q4_0 || KT == KVQ_Q5_0) c = b, within = 4 * j;
            else c = 4 * b + j, within = 0;
            k_rd[T][b] = g::K_OFF + (r * g::CPR + (c ^ kswz<g::CPR>(r))) * 16 + within;
        }
    }
    constexpr bool VNIB = VT == KVQ_Q4_0 || VT == KVQ_Q5_0;  // nibble-packed V
    constexpr int VL = (VNIB || VT == KVQ_TURBO3) ? NB : NCT;  // V operand reads per tile
    int v_rd[VL];
#pragma unroll
    for (int i = 0; i < VL; i++) {
        // q4_0 / q5_0: byte n of block i; turbo3: byte n&7 of block i; else channel 16i+n
        const int u = (VT == KVQ_TURBO3) ? 8 * i + (n & 7) : 16 * i + n;
        const int c = (VT == KVQ_F16) ? u : (u >> 1);
        const int within = (VT == KVQ_F16) ? 0 : 8 * (u & 1);
        v_rd[i] = g::V_OFF + (j * g::CPG + (c ^ vswz<VT, g::CPG>(j))) * 16 + within;
    }

    float m_run;    // running max (base 2) of head n, equal in the 4 lane groups
    float l_run;    // this lane's share of the running sum
    floatx4 o[NCT];
    auto reset = [&]() {
        m_run = -INFINITY;
        l_run = 0.0f;
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
            o[ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    };

    // The operands of one tile, read from its LDS copy into registers.
    struct Ops {
        u32x4 k[2][NB];                 // K codes per S-tile and block (words used by the type)
        uint32_t ks[4 * NB];            // K scales: token r, block b at half r*NB+b
        u32x4 v[VL];                    // V codes per read
        u32x4 vs[NB];                   // V scales: block b, tokens 0..7
        uint32_t kh[KT == KVQ_Q5_0 ? 2 : 1][KT == KVQ_Q5_0 ? NB : 1];     // q5_0 K high bits
        uint32_t vh[has_bit_words(VT) ? NB : 1][has_bit_words(VT) ? 8 : 1];  // V high / third bits, tokens 0..7
    };
    auto read_ops = [&](const uint8_t *buf, Ops &op) {
#pragma unroll
        for (int T = 0; T < 2; T++)
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (KT == KVQ_F16) {
                    op.k[T][b] = *reinterpret_cast<const u32x4 *>(buf + k_rd[T][b]);
                } else if (KT == KVQ_Q8_0) {
                    const u32x2 w = *reinterpret_cast<const u32x2 *>(buf + k_rd[T][b]);
                    op.k[T][b] = u32x4{w.x, w.y, 0u, 0u};
                } else {
                    op.k[T][b] = u32x4{*reinterpret_cast<const uint32_t *>(buf + k_rd[T][b]), 0u, 0u, 0u};
                }
            }
        if (KT != KVQ_F16) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(buf + g::KS_OFF + 16 * NB * j);
#pragma unroll
            for (int i = 0; i < NB; i++) {
                const u32x4 w = p[i];
                op.ks[4 * i] = w.x, op.ks[4 * i + 1] = w.y, op.ks[4 * i + 2] = w.z, op.ks[4 * i + 3] = w.w;
            }
        }
#pragma unroll
        for (int i = 0; i < VL; i++) {
            if (VT == KVQ_F16) {
                op.v[i] = *reinterpret_cast<const u32x4 *>(buf + v_rd[i]);
            } else {
                const u32x2 w = *reinterpret_cast<const u32x2 *>(buf + v_rd[i]);
                op.v[i] = u32x4{w.x, w.y, 0u, 0u};
            }
        }
        if (VT != KVQ_F16) {
#pragma unroll
            for (int b = 0; b < NB; b++)
                op.vs[b] = *reinterpret_cast<const u32x4 *>(buf + g::VS_OFF + (j * NB + b) * 16);
        }
        if constexpr (KT == KVQ_Q5_0) {
#pragma unroll
            for (int T = 0; T < 2; T++) {
                const int r = 8 * (n >> 2) + 4 * T + (n & 3);
#pragma unroll
                for (int b = 0; b < NB; b++)
                    op.kh[T][b] = *reinterpret_cast<const uint32_t *>(buf + g::KH_OFF + (r * NB + b) * 4);
            }
        }
        if constexpr (has_bit_words(VT)) {
#pragma unroll
            for (int b = 0; b < NB; b++) {
                const u32x4 *p = reinterpret_cast<const u32x4 *>(buf + g::VH_OFF + (j * NB + b) * 32);
                const u32x4 w0 = p[0], w1 = p[1];
                op.vh[b][0] = w0.x, op.vh[b][1] = w0.y, op.vh[b][2] = w0.z, op.vh[b][3] = w0.w;
                op.vh[b][4] = w1.x, op.vh[b][5] = w1.y, op.vh[b][6] = w1.z, op.vh[b][7] = w1.w;
            }
        }
    };

    // One 32-token tile starting at token tb, from its operands in registers.
    auto process = [&](Ops &op, const int tb, const int t_end) {
        // ---------------- scores: S^T tile T, lane holds tokens 8j+4T+i, head n
        const uint32_t *ksc = op.ks;
        floatx4 sacc[2];
#pragma unroll
        for (int T = 0; T < 2; T++) {
            sacc[T] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int b = 0; b < NB; b++) {
                half8 ka;
                if constexpr (KT == KVQ_F16) {
                    const u32x4 w = op.k[T][b];
                    ka = pack4(w.x, w.y, w.z, w.w);
                } else if constexpr (KT == KVQ_Q8_0) {
                    ka = deq_q8_sub(op.k[T][b].x, op.k[T][b].y);
                } else if constexpr (KT == KVQ_Q4_0) {
                    ka = k_operand_q4_sub(op.k[T][b].x);
                } else {
                    ka = k_operand_q4_sub(op.k[T][b].x);  // the nibbles; the fifth bits below
                }
                if (KT == KVQ_F16) {
                    sacc[T] = mfma(ka, qb[b], sacc[T]);
                } else {
                    floatx4 c = mfma(ka, qb[b], KSUB ? kofs[KSUB ? b : 0] : floatx4{0.0f, 0.0f, 0.0f, 0.0f});
                    if constexpr (K5)
                        c = mfma(k_operand_q5_fifth(op.kh[T][b], j), qb5[K5 ? b : 0], c);
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        sacc[T][i] = __builtin_fmaf(half_at(ksc, (4 * T + i) * NB + b), c[i], sacc[T][i]);
                }
            }
        }

        // ---------------- online softmax (base 2); token r of group j is tb+8j+r
        float x[8];
#pragma unroll
        for (int r = 0; r < 8; r++)
            x[r] = sacc[r >> 2][r & 3] * c2;
        // The tile past the context (at most one per wave, its last): masked
        // tokens' scores become -inf, and since positions past the context
        // may hold any bits, their V scales (binary16 V: their values) are
        // forced to +0, so that P' = p * scale is +0 rather than 0 * NaN.
        // Only this branch pays for the masks.
        if (tb + TILE > t_end) {
            uint32_t keep[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};  // per token pair
#pragma unroll
            for (int r = 0; r < 8; r++)
                if (tb + 8 * j + r >= t_end) {
                    x[r] = -INFINITY;
                    keep[r >> 1] &= (r & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                }
            if (VT == KVQ_F16) {
#pragma unroll
                for (int ct = 0; ct < VL; ct++)
                    op.v[ct] = u32x4{op.v[ct].x & keep[0], op.v[ct].y & keep[1], op.v[ct].z & keep[2], op.v[ct].w & keep[3]};
            } else {
#pragma unroll
                for (int b = 0; b < NB; b++)
                    op.vs[b] = u32x4{op.vs[b].x & keep[0], op.vs[b].y & keep[1], op.vs[b].z & keep[2], op.vs[b].w & keep[3]};
            }
        }
        const float mt = max_lane_groups(max3(max3(x[0], x[1], x[2]), max3(x[3], x[4], x[5]), max3(x[6], x[7], x[7])));
        if (__any(mt > m_run)) {
            const float m_new = __builtin_elementwise_maximum(m_run, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
            l_run *= alpha;
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
                o[ct] *= alpha;
            m_run = m_new;
        }
        float p[8];
#pragma unroll
        for (int r = 0; r < 8; r++) {
            p[r] = __builtin_amdgcn_exp2f(x[r] - m_run);
            l_run += p[r];
        }
        // binary16 probabilities, token pairs (0,1) (2,3) (4,5) (6,7)
        uint32_t p16[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            p16[i] = h2_bits(__builtin_convertvector((float2v){p[2 * i], p[2 * i + 1]}, half2));

        // ---------------- O^T += V^T . P'
#pragma unroll
        for (int b = 0; b < NB; b++) {
            half8 pb;  // P' of block b in k-slot order = token order 0..7
            if (VT == KVQ_F16) {
                pb = pack4(p16[0], p16[1], p16[2], p16[3]);
            } else {
                const u32x4 dv = op.vs[b];  // masked tokens' scales are +0 (tail tile)
                pb = pack4(h2_bits(bits_h2(p16[0]) * bits_h2(dv.x)), h2_bits(bits_h2(p16[1]) * bits_h2(dv.y)),
                           h2_bits(bits_h2(p16[2]) * bits_h2(dv.z)), h2_bits(bits_h2(p16[3]) * bits_h2(dv.w)));
            }
            if constexpr (VT == KVQ_Q4_0) {
                // bytes of tokens 0..3 (word 0) and 4..7 (word 1); low nibbles feed
                // channel tile 2b (c * 2^-24), high nibbles tile 2b+1 (16 c *
                // 2^-24); the offset 8 (16 * 8) comes off by one more MFMA each
                half8 va0, va1;
                v_operand_q4_sub(u32x2{op.v[b].x, op.v[b].y}, va0, va1);
                o[2 * b] = mfma(va0, pb, o[2 * b]);
                o[2 * b + 1] = mfma(va1, pb, o[2 * b + 1]);
                o[2 * b] = mfma(pack4(SUB_NEG8, SUB_NEG8, SUB_NEG8, SUB_NEG8), pb, o[2 * b]);
                o[2 * b + 1] = mfma(pack4(SUB_NEG128, SUB_NEG128, SUB_NEG128, SUB_NEG128), pb, o[2 * b + 1]);
            } else if constexpr (VT == KVQ_Q5_0) {
                // as q4_0, each code's fifth bit from its token's high-bit word
                half8 va0, va1;
                v_operand_q5(u32x2{op.v[b].x, op.v[b].y}, op.vh[b], n, va0, va1);
                o[2 * b] = mfma(va0, pb, o[2 * b]);
                o[2 * b + 1] = mfma(va1, pb, o[2 * b + 1]);
            } else if constexpr (VT == KVQ_TURBO3) {
                // codebook levels of the rotated values: O accumulates in the
                // rotated basis, the merge rotates it back
                half8 va0, va1;
                v_operand_tq3(u32x2{op.v[b].x, op.v[b].y}, op.vh[b], n, va0, va1);
                o[2 * b] = mfma(va0, pb, o[2 * b]);
                o[2 * b + 1] = mfma(va1, pb, o[2 * b + 1]);
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    const int ct = 2 * b + hh;
                    half8 va;
                    const u32x4 w = op.v[ct];
                    if (VT == KVQ_F16) {
                        va = pack4(w.x, w.y, w.z, w.w);  // masked tokens' values are +0 (tail tile)
                    } else {
                        va = deq_q8_sub(w.x, w.y);  // (c + 128) * 2^-24
                    }
                    o[ct] = mfma(va, pb, o[ct]);
                }
                if (VT == KVQ_Q8_0) {
#pragma unroll
                    for (int hh = 0; hh < 2; hh++)
                        o[2 * b + hh] = mfma(pack4(SUB_NEG128, SUB_NEG128, SUB_NEG128, SUB_NEG128), pb, o[2 * b + hh]);
                }
            }
        }
    };

    // ---------------- stream the wave's tiles.  Per tile: wait for its copy,
    // read its operands out of LDS into registers, start the copy of a later
    // tile into the freed LDS space, then compute.  With NBUF LDS buffers per
    // wave the copies of the next NBUF tiles are in flight during the math of
    // the current one.
    //
    // The waits are explicit: the compiler does not reliably track
    // direct-to-LDS copies against LDS reads.  Vector-memory loads complete
    // in issue order, so "at most n*NDMA outstanding" (NDMA = the count of
    // one tile's copy instructions) means every load issued before the n
    // newer tiles' copies has completed.
    constexpr int NDMA = g::NDMA;
    static_assert((NBUF - 1) * NDMA < 64, "vmcnt holds 6 bits");
    // s_waitcnt immediate for vmcnt(n * NDMA), expcnt and lgkmcnt untouched
    auto wait_imm = [](int n) constexpr { return ((n * NDMA) & 15) | (((n * NDMA) >> 4) << 14) | 0x70 | 0xF00; };
    auto wait_newer = [&](const int newer) __attribute__((always_inline)) {
        // at most `newer` tiles' copies may still be outstanding
        static_for<NBUF>([&](auto c) {
            if (newer == c)
                __builtin_amdgcn_s_waitcnt(wait_imm(c));
        });
    };

    reset();
    // Tile i (of n_mine) sits in `buf`; the copies of tiles i+1 .. i+NBUF-1
    // (those below n_mine) were issued after it; tile i+NBUF goes into `buf`
    // once tile i's operands are in registers.
    auto step = [&](uint8_t *buf, const int i) __attribute__((always_inline)) {
        wait_newer(min(NBUF - 1, n_mine - 1 - i));
        Ops op;
        read_ops(buf, op);
        if (i + NBUF < n_mine) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS reads done before it is refilled
            issue_tile<KT, VT, D, CPOL_STREAM>(buf, (r + (i + NBUF) * k) * TILE, lane, doff, rs);
        }
        process(op, (r + i * k) * TILE, ctx);
    };
    static_for<NBUF>([&](auto u) {  // an idle wave (r >= k, n_mine = 0) streams nothing
        if (u < n_mine)
            issue_tile<KT, VT, D, CPOL_STREAM>(lds_t[u] + wave * g::BYTES, (r + u * k) * TILE, lane, doff, rs);
    });
    // the query operands' block sums and slot order (see where qb is loaded),
    // once the first copies are on their way
    if constexpr (KSUB) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            float qs = 0.0f;  // the lane's 8 channels, then the four lane groups
#pragma unroll
            for (int r = 0; r < 8; r++)
                qs += (float)qb[b][r];
            qs += __shfl_xor(qs, 16);
            qs += __shfl_xor(qs, 32);
            const float o = (KT == KVQ_Q8_0 ? -128.0f : KT == KVQ_Q5_0 ? -16.0f : -8.0f) * TWO_M24 * qs;
            kofs[b] = floatx4{o, o, o, o};
            if constexpr (K5) {
                // fifth-bit slots 2k, 2k+1: elements 4j+k and 16+4j+k, times 2^-k
                const u32x4 w = __builtin_bit_cast(u32x4, qb[b]);
                const half2 s1 = {(_Float16)1.0f, (_Float16)1.0f}, s2 = {(_Float16)0.5f, (_Float16)0.5f};
                const half2 s4 = {(_Float16)0.25f, (_Float16)0.25f}, s8 = {(_Float16)0.125f, (_Float16)0.125f};
                qb5[K5 ? b : 0] = pack4(h2_bits(bits_h2(__builtin_amdgcn_perm(w.z, w.x, 0x05040100u)) * s1),
                                        h2_bits(bits_h2(__builtin_amdgcn_perm(w.z, w.x, 0x07060302u)) * s2),
                                        h2_bits(bits_h2(__builtin_amdgcn_perm(w.w, w.y, 0x05040100u)) * s4),
                                        h2_bits(bits_h2(__builtin_amdgcn_perm(w.w, w.y, 0x07060302u)) * s8));
            }
            if constexpr (KT == KVQ_Q4_0 || KT == KVQ_Q5_0) {
                // slots: elements 4j, 4j+2, 4j+1, 4j+3, then the high
                // nibbles' 16+4j, ... scaled by 1/16
                const u32x4 w = __builtin_bit_cast(u32x4, qb[b]);
                const half2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
                qb[b] = pack4(__builtin_amdgcn_perm(w.y, w.x, 0x05040100u), __builtin_amdgcn_perm(w.y, w.x, 0x07060302u),
                              h2_bits(bits_h2(__builtin_amdgcn_perm(w.w, w.z, 0x05040100u)) * k16),
                              h2_bits(bits_h2(__builtin_amdgcn_perm(w.w, w.z, 0x07060302u)) * k16));
            }
        }
    }
    int i = 0;
    for (; i + NBUF <= n_mine; i += NBUF)
        static_for<NBUF>([&](auto u) { step(lds_t[u] + wave * g::BYTES, i + u); });
    static_for<NBUF - 1>([&](auto u) {  // the last n_mine mod NBUF tiles, in buffers 0, 1, ...
        if (i < n_mine) {
            step(lds_t[u] + wave * g::BYTES, i);
            i++;
        }
    });

    // Subnormal value operands: O back to its units (q8_0: 2^24; q4_0: 2^24
    // for the low nibbles' channel tiles 2b, 2^20 for the high nibbles' tiles
    // 2b+1, which summed 16 c).
    if constexpr (VT == KVQ_Q8_0 || VT == KVQ_Q4_0) {
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
            o[ct] *= (VT == KVQ_Q4_0 && (ct & 1)) ? 1048576.0f : TWO_P24;
    }

    // ---------------- merge the workgroup's four partials in LDS.  Lane
    // (n, j) holds head n's running max m_run (base 2, equal in the four lane
    // groups), its share l_run of the running sum, and O of channels
    // 16ct + 4j + i.  Waves with no tiles hold m = -inf, l = 0, O = 0; wave
    // 0 always has tiles (4 rw < k), so every head's maximum is finite.
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    __syncthreads();  // every wave has left its tile loop: lds_a is free
    float *const ml = reinterpret_cast<float *>(lds_a);        // [wave][m: 16 | l: 16]
    float *const acc = ml + WAVES * 32;                        // [G][D]: running sum of the scaled O
    if (j == 0) {
        ml[wave * 32 + n] = m_run;
        ml[wave * 32 + 16 + n] = l_tot;
    }
    __syncthreads();
    float M = ml[n];
#pragma unroll
    for (int w = 1; w < WAVES; w++)
        M = fmaxf(M, ml[w * 32 + n]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; w++)  // fixed order: results do not depend on timing
        L += ml[w * 32 + 16 + n] * __builtin_amdgcn_exp2f(ml[w * 32 + n] - M);
    const float f = __builtin_amdgcn_exp2f(m_run - M);
#pragma unroll
    for (int ct = 0; ct < NCT; ct++)
        o[ct] *= f;
    // O summed over the waves in wave order; the last wave keeps the sum
    floatx4 *const accv = reinterpret_cast<floatx4 *>(acc + n * D + 4 * j);
#pragma unroll
    for (int w = 0; w < WAVES; w++) {
        if (wave == w && n < G) {
#pragma unroll
            for (int ct = 0; ct < NCT; ct++) {
                if (w > 0)
                    o[ct] += accv[4 * ct];
                if (w < WAVES - 1)
                    accv[4 * ct] = o[ct];
            }
        }
        if (w < WAVES - 1)
            __syncthreads();
    }

    float *const out = a.out + ((int64_t)s * a.Hq + (int64_t)h * G) * D;
    if (kw == 1) {
        // the pair's only workgroup: normalize and write the output
        if (wave == WAVES - 1) {
            const float inv = 1.0f / L;
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
                o[ct] *= inv;
            if constexpr (VT == KVQ_TURBO3)
                rotate_back_tiles<NCT>(o, lane);  // O was accumulated in the rotated basis
            if (n < G) {
#pragma unroll
                for (int ct = 0; ct < NCT; ct++)
                    *reinterpret_cast<floatx4 *>(out + n * D + 16 * ct + 4 * j) = o[ct];
            }
        }
        return;
    }

    // ---------------- several workgroups: write this one's slot (O, m, l per
    // head) with device-coherent stores, count in, and let the last one merge
    const int SL = G * (D + 4);  // floats per slot
    float *const slots = a.ws;
    uint32_t *const counter = a.counters + pair;
    if (wave == WAVES - 1) {
        if (n < G) {
            const __amdgpu_buffer_rsrc_t rw_ = make_rsrc(slots + (int64_t)(slot0 + rw * slot_step) * SL, SL * 4);
            const int off = 4 * (n * (D + 4) + 4 * j);
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[ct]), rw_, off + 64 * ct, 0,
                                                       CPOL_SC1);
            if (j == 0) {
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, M), rw_, off + 4 * D, 0, CPOL_SC1);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, L), rw_, off + 4 * D + 4, 0,
                                                      CPOL_SC1);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the slot is written before the count
        if (lane == 0)
            mrg_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       (uint32_t)(kw - 1);
    }
    __syncthreads();
    if (!mrg_last)
        return;

    // ---------------- the last workgroup of the pair: combine its kw slots
    // (device-coherent loads; slot order).  Weights w_jg = 2^(m_jg - M_g) and
    // sums L_g = sum_j l_jg w_jg per head g, then each thread sums O of its
    // (head, channel) outputs with those weights.
    const int t = threadIdx.x;
    const int nw = kw * G;
    float *const mrg_w = reinterpret_cast<float *>(lds_a);  // the workgroup merge's data is no longer read
    float *const mrg_l = mrg_w + MERGE_SLOTS;
    auto slot_ptr = [&](int jj) { return slots + (int64_t)(slot0 + jj * slot_step) * SL; };
    // One thread per (slot, head) entry e = jj * G + gg (at most EPT per
    // thread): its weight 2^(m_e - M_gg) and its scaled sum l_e * weight, all
    // entries at once -- no thread walks the slots one dependent LDS read
    // after another.
    constexpr int EPT = (MERGE_SLOTS + 64 * WAVES - 1) / (64 * WAVES);
    float me[EPT], le[EPT];
#pragma unroll
    for (int u = 0; u < EPT; u++) {
        const int e = t + u * 64 * WAVES;
        if (e < nw) {
            const int jj = e / G, gg = e - jj * G;
            const float *p = slot_ptr(jj) + gg * (D + 4) + D;
            me[u] = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            le[u] = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            mrg_w[e] = me[u];
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < EPT; u++) {
        const int e = t + u * 64 * WAVES;
        if (e < nw) {
            const int gg = e % G;
            float M = mrg_w[gg];
#pragma unroll 8
            for (int jj = 1; jj < kw; jj++)
                M = fmaxf(M, mrg_w[jj * G + gg]);
            me[u] = __builtin_amdgcn_exp2f(me[u] - M);
            le[u] *= me[u];
        }
    }
    __syncthreads();  // every maximum is read before the weights replace the maxima
#pragma unroll
    for (int u = 0; u < EPT; u++) {
        const int e = t + u * 64 * WAVES;
        if (e < nw) {
            mrg_w[e] = me[u];
            mrg_l[e] = le[u];
        }
    }
    __syncthreads();
    // Outputs in quads of channels: thread t sums channels 4q .. 4q+3 of one
    // head for quads q = t, t + 256, ... (D/4 quads per head), one 16-byte
    // load per slot, all the slots' loads of a quad issued together.  Eight
    // consecutive threads hold one 32-channel block (turbo3's rotation back).
    const int nq = G * D / 4;
    // a descriptor per slot (the slot bases are wave-uniform; the slots of one
    // pair may lie further apart than 32-bit buffer offsets reach)
    auto slot_rsrc = [&](int jj) { return make_rsrc(slots + (int64_t)(slot0 + jj * slot_step) * SL, SL * 4); };
    for (int qd = t; qd < (nq + 63) / 64 * 64; qd += 64 * WAVES) {  // whole waves (rotation shuffles)
        const bool live = qd < nq;
        const int gg = live ? qd / (D / 4) : 0, c = 4 * (qd - gg * (D / 4));
        const int off = 4 * (gg * (D + 4) + c);
        floatx4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
        if (live) {
            float L = 0.0f;  // the head's sum over the slots, in slot order
#pragma unroll 8
            for (int j2 = 0; j2 < kw; j2++)
                L += mrg_l[j2 * G + gg];
            int jj = 0;
            for (; jj + 16 <= kw; jj += 16) {  // sixteen loads in flight, summed in slot order
                floatx4 v[16];
#pragma unroll
                for (int u = 0; u < 16; u++)
                    v[u] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(slot_rsrc(jj + u), off, 0,
                                                                                             CPOL_SC1));
#pragma unroll
                for (int u = 0; u < 16; u++)
                    sum += v[u] * mrg_w[(jj + u) * G + gg];
            }
            for (; jj < kw; jj++)
                sum += __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(slot_rsrc(jj), off, 0, CPOL_SC1)) *
                       mrg_w[jj * G + gg];
            sum *= 1.0f / L;
        }
        if constexpr (VT == KVQ_TURBO3)
            sum = rotate_back_quad(sum, c);
        if (live)
            *reinterpret_cast<floatx4 *>(out + gg * D + c) = sum;
    }
    if (t == 0)  // the next call on this workspace starts from zero again
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int KT, int VT, int D>
hipError_t launch_dec(const DecodeArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL((decode_kernel<KT, VT, D>), dim3(a.n_wg), dim3(64 * WAVES), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dec_d(int kt, int vt, const DecodeArgs &a, hipStream_t st)
{
#define KVQ_D(K, V) \
    if (kt == K && vt == V) return launch_dec<K, V, D>(a, st);
    KVQ_FOR_EACH_TYPE_PAIR(KVQ_D)
#undef KVQ_D
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(int kt, int vt, int D, const DecodeArgs &a, hipStream_t st)
{
    switch (D) {
    case 64: return launch_dec_d<64>(kt, vt, a, st);
    case 128: return launch_dec_d<128>(kt, vt, a, st);
    case 256: return launch_dec_d<256>(kt, vt, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
