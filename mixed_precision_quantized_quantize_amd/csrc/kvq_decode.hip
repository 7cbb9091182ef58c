// kvq_decode.hip -- flash decode over the quantized cache: one persistent
// streaming kernel and one log-sum-exp merge kernel.
//
// Flash attention in the sense of the llama.cpp guide's "Flash Attention"
// section (tiled, the score matrix never materialized, exactly softmax
// attention), reading the quantized blocks directly -- the KVSplit page's
// discussion expects the gain "integrated directly into FlashAttention", and
// the llama.cpp issue shows a quantized V cache is only usable that way.
//
// Work split.  Every (sequence, kv head) pair gets k waves (k per sequence,
// about proportional to its context, at least one tile per wave); wave r of
// a pair takes the pair's 32-token tiles r, r+k, r+2k, ... so that the k
// waves stream neighbouring tiles at any moment.  Each wave writes one
// partial -- running max m (base 2), sum l and the unnormalized output O of
// each query head -- into its own slot, and the merge kernel combines the k
// partials of each pair.  A wave keeps the copies of its next two tiles in
// flight while it computes the current one.
//
// Per tile a wave serves the whole GQA group (up to 16 query heads) of its kv
// head with two matrix-core contractions, both v_mfma_f32_16x16x32_f16:
//   S^T[token][head] = K[token][c] . Q^T[c][head]  -- one MFMA per 16 tokens
//       and 32-channel block; the raw codes are exact in binary16 and the
//       block's K scale multiplies the MFMA result per token;
//   O^T[chan][head] += V^T[chan][token] . P'[token][head]  -- one MFMA per 16
//       channels and 32 tokens; P' = binary16(p) * V scale of (token, block).
// The score layout of the first product is exactly the operand layout of the
// second, so probabilities never leave registers.  The V plane stores 8
// tokens interleaved, so a lane's P.V operand (8 tokens of one channel) is
// one 8- or 16-byte load.  Online softmax runs in base 2 (scores times
// scale*log2 e).
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
    while (n > 1 && (n * g::LDS_A > 160 * 1024 || (n - 1) * NDMA >= 64))
        n--;
    return n;
}

template <int KT, int VT, int D>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1))) void decode_kernel(const DecodeArgs a)
{
    using g = Geo<KT, VT, D>;
    constexpr int NB = g::NB, NCT = g::NCT;

    // NBUF tile buffers per wave, as many as fit (up to KVQ_DECODE_NBUF), in
    // separate arrays so that the compiler sees that a read of one does not
    // wait for another
    constexpr int NBUF = decode_nbuf<KT, VT, D>();
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[g::LDS_A];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[NBUF >= 2 ? g::LDS_A : 16];
    __shared__ __attribute__((aligned(16))) uint8_t lds_c[NBUF >= 3 ? g::LDS_A : 16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
    const int n = lane & 15, j = lane >> 4;
    const int gw = blockIdx.x * WAVES + wave;
    if (gw >= a.W)
        return;
    const int G = a.G, Hkv = a.Hkv;
    const int64_t Tc = a.Tc;

    // this wave's pair (s, h) and its index r among the pair's k waves.
    // The pairs are interleaved over the grid (wave gw serves pair
    // gw mod pairs), so that every pair gets waves from early- and
    // late-dispatched workgroups alike: with two workgroups per CU the first
    // one on a CU runs well ahead of the second, and pairs served by only one
    // of them would finish far apart.  When every sequence has k waves per
    // pair this is a division; else the sequences' first waves are binary
    // searched (dependent scalar loads) and the heads of one sequence are
    // interleaved.
    int s = 0, k = a.k_uniform, h, r;
    if (k > 0) {
        const int n_pairs = a.n_seqs * Hkv;
        r = gw / n_pairs;
        const int pg = gw - r * n_pairs;
        s = pg / Hkv;
        h = pg - s * Hkv;
    } else {
        int hi = a.n_seqs;  // wave_start[s] <= gw < wave_start[hi]
        while (hi - s > 1) {
            const int mid = (s + hi) >> 1;
            if (a.wave_start[mid] <= gw)
                s = mid;
            else
                hi = mid;
        }
        k = (a.wave_start[s + 1] - a.wave_start[s]) / Hkv;
        const int local = gw - a.wave_start[s];
        r = local / Hkv;
        h = local - r * Hkv;
    }
    const int ctx = a.ctx_len[s];
    const int nt = (ctx + TILE - 1) / TILE;
    const int n_mine = (nt - r + k - 1) / k;  // tiles r, r+k, ... below nt (>= 1)
    const int64_t pair = (int64_t)s * Hkv + h;

    // Fused one-row append: the wave that reads the pair's last tile first
    // quantizes the new row into position ctx-1 (one quad of lanes per
    // 32-element block, K blocks then V blocks, the append kernel's
    // quantizer), and waits until the stores are performed before any copy
    // of that tile is issued.  No other wave reads that tile.
    if (a.knew != nullptr && r == (nt - 1) % k) {
        const int quad = lane >> 2, q = lane & 3;
        if (quad < 2 * NB) {
            const int role = quad >= NB, b = quad - role * NB;
            const uint16_t *blk = (role ? a.vnew : a.knew) + pair * D + 32 * b;
            if (role == 0)
                quant::quant_store<KT, 0>(blk, q, const_cast<uint8_t *>(a.kc), const_cast<uint16_t *>(a.ks),
                                          const_cast<uint32_t *>(a.kqh), pair, ctx - 1, b, D, a.Tc);
            else
                quant::quant_store<VT, 1>(blk, q, const_cast<uint8_t *>(a.vc), const_cast<uint16_t *>(a.vs),
                                          const_cast<uint32_t *>(a.vqh), pair, ctx - 1, b, D, a.Tc);
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

    // Q^T operand: lane (n = head, j) holds 8 channels of each block (the
    // channels qk_chan picks: 8j.. for f16/q8_0, 4j.. and 16+4j.. for q4_0);
    // buffer loads from the scalar base of the pair's Q rows
    half8 qb[NB];
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
    const float c2 = a.c2;

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

    const int bp16 = (lane ^ 16) << 2, bp32 = (lane ^ 32) << 2;  // ds_bpermute byte addresses
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
                    ka = deq_q8(op.k[T][b].x, op.k[T][b].y);
                } else if constexpr (KT == KVQ_Q4_0) {
                    const uint32_t w = op.k[T][b].x;
                    ka = k_operand<KVQ_Q4_0>(&w);
                } else {
                    ka = k_operand_q5(op.k[T][b].x, op.kh[T][b] >> (4 * j));
                }
                if (KT == KVQ_F16) {
                    sacc[T] = mfma(ka, qb[b], sacc[T]);
                } else {
                    const floatx4 c = mfma(ka, qb[b], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
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
        float mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mt = fmaxf(mt, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp16, __builtin_bit_cast(int, mt))));
        mt = fmaxf(mt, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp32, __builtin_bit_cast(int, mt))));
        if (__any(mt > m_run)) {
            const float m_new = fmaxf(m_run, mt);
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
                // channel tile 2b, high nibbles tile 2b+1
                const u32x4 w = op.v[b];
                uint32_t l01, h01, l23, h23, l45, h45, l67, h67;
                deq_q4_pair(__builtin_amdgcn_perm(w.x, w.x, 0x0C010C00u), l01, h01);
                deq_q4_pair(__builtin_amdgcn_perm(w.x, w.x, 0x0C030C02u), l23, h23);
                deq_q4_pair(__builtin_amdgcn_perm(w.y, w.y, 0x0C010C00u), l45, h45);
                deq_q4_pair(__builtin_amdgcn_perm(w.y, w.y, 0x0C030C02u), l67, h67);
                o[2 * b] = mfma(pack4(l01, l23, l45, l67), pb, o[2 * b]);
                o[2 * b + 1] = mfma(pack4(h01, h23, h45, h67), pb, o[2 * b + 1]);
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
                        va = deq_q8(w.x, w.y);
                    }
                    o[ct] = mfma(va, pb, o[ct]);
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
    constexpr int WAIT_ALL = 0x70 | 0xF00;  // vmcnt(0), expcnt and lgkmcnt untouched
    constexpr int WAIT_1 = (NDMA & 15) | ((NDMA >> 4) << 14) | 0x70 | 0xF00;                    // vmcnt(NDMA)
    constexpr int WAIT_2 = ((2 * NDMA) & 15) | (((2 * NDMA) >> 4) << 14) | 0x70 | 0xF00;        // vmcnt(2*NDMA)

    reset();
    // Tile i (of n_mine) sits in `buf`; the copies of tiles i+1 .. i+NBUF-1
    // (those below n_mine) were issued after it; tile i+NBUF goes into `buf`
    // once tile i's operands are in registers.
    auto step = [&](uint8_t *buf, const int i) {
        const int newer = min(NBUF - 1, n_mine - 1 - i);
        if (NBUF >= 3 && newer >= 2)
            __builtin_amdgcn_s_waitcnt(WAIT_2);
        else if (NBUF >= 2 && newer >= 1)
            __builtin_amdgcn_s_waitcnt(WAIT_1);
        else
            __builtin_amdgcn_s_waitcnt(WAIT_ALL);
        Ops op;
        read_ops(buf, op);
        if (i + NBUF < n_mine) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS reads done before it is refilled
            issue_tile<KT, VT, D, CPOL_STREAM>(buf, (r + (i + NBUF) * k) * TILE, lane, doff, rs);
        }
        process(op, (r + i * k) * TILE, ctx);
    };
    uint8_t *const buf_a = lds_a + wave * g::BYTES;
    uint8_t *const buf_b = lds_b + wave * g::BYTES;
    uint8_t *const buf_c = lds_c + wave * g::BYTES;
    issue_tile<KT, VT, D, CPOL_STREAM>(buf_a, r * TILE, lane, doff, rs);
    if (NBUF >= 2 && n_mine > 1)
        issue_tile<KT, VT, D, CPOL_STREAM>(buf_b, (r + k) * TILE, lane, doff, rs);
    if (NBUF >= 3 && n_mine > 2)
        issue_tile<KT, VT, D, CPOL_STREAM>(buf_c, (r + 2 * k) * TILE, lane, doff, rs);
    int i = 0;
    for (; i + NBUF <= n_mine; i += NBUF) {
        step(buf_a, i);
        if constexpr (NBUF >= 2)
            step(buf_b, i + 1);
        if constexpr (NBUF >= 3)
            step(buf_c, i + 2);
    }
    if (NBUF >= 2 && i < n_mine)
        step(buf_a, i++);
    if (NBUF >= 3 && i < n_mine)
        step(buf_b, i++);

    // ---------------- the wave's partial: O of head n (channels 16ct + 4j + i),
    // m, l -- buffer stores from the scalar base of the slot
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (n < G) {
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.ws + (int64_t)gw * G * (D + 4), G * (D + 4) * 4);
        const int off = 4 * (n * (D + 4) + 4 * j);
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[ct]), rw, off + 64 * ct, 0, 0);
        if (j == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, m_run), rw, off + 4 * D, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l_tot), rw, off + 4 * D + 4, 0, 0);
        }
    }
}

// Log-sum-exp merge of the partials of one (sequence, kv head) pair for one
// query head: workgroup = (pair, head), P groups of one thread per output
// channel.  The slot weights 2^(m_j - M) go through LDS in chunks; group p
// sums slots p, p+P, ... of a chunk, up to sixteen independent loads at a time, and
// the groups' sums are added through LDS at the end.  P grows with the
// slots per pair so that a long merge is not one thread's chain of loads.
constexpr int MERGE_CHUNK = 512;
constexpr int MERGE_MAX_THREADS = 1024;

__device__ inline float block_reduce(float v, float *sh, bool is_max)
{
    // wave64 butterfly, then across the waves of the workgroup through LDS
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float u = __shfl_xor(v, o);
        v = is_max ? fmaxf(v, u) : v + u;
    }
    const int wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        sh[wave] = v;
    __syncthreads();
    float r = sh[0];
    for (int w = 1; w < nw; w++)
        r = is_max ? fmaxf(r, sh[w]) : r + sh[w];
    return r;
}

// turbo3 values: rotate each 32-channel block of the output back,
// x = s.(H y)/32 -- butterflies of span 1..16 across the 32 threads (lanes)
// of the block, thread c holding channel c
__device__ inline float rotate_back(float r, const int c)
{
#pragma unroll
    for (int span = 1; span < 32; span <<= 1) {
        const float o = __shfl_xor(r, span);
        r = (c & span) ? o - r : r + o;
    }
    return ((TQ3_SIGNS >> (c & 31)) & 1u) ? -r * 0.03125f : r * 0.03125f;
}

// Channel c of one query head from its k <= KF partials (slot j at
// base + j*stride): all 3*KF loads issued together (slots past k repeat the
// last one and weigh nothing), then sum_j O_j[c] 2^(m_j - M) / sum_j l_j 2^(m_j - M)
// in slot order.
template <int KF>
__device__ inline float merge_few(const float *base, const int64_t stride, const int k, const int c, const int D)
{
    float mj[KF], lj[KF], oj[KF];
#pragma unroll
    for (int j = 0; j < KF; j++) {
        const float *pk = base + (int64_t)min(j, k - 1) * stride;
        mj[j] = pk[D];
        lj[j] = pk[D + 1];
        oj[j] = pk[c];
    }
    float M = mj[0];
#pragma unroll
    for (int j = 1; j < KF; j++)
        if (j < k)
            M = fmaxf(M, mj[j]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int j = 0; j < KF; j++)
        if (j < k) {
            const float w = __builtin_amdgcn_exp2f(mj[j] - M);
            L += lj[j] * w;
            acc += oj[j] * w;
        }
    return acc / L;
}

__global__ __launch_bounds__(MERGE_MAX_THREADS) void merge_kernel(const MergeArgs a)
{
    __shared__ float wts[MERGE_CHUNK];
    __shared__ float red[MERGE_MAX_THREADS / 64];
    __shared__ float part[MERGE_MAX_THREADS];
    const int G = a.G, D = a.D, Dp = a.D + 4;
    const int P = blockDim.x / D;  // groups; blockDim.x == P * D
    const int pair = blockIdx.x / G, gg = blockIdx.x - pair * G;
    const int s = pair / a.Hkv, h = pair - s * a.Hkv;
    const int k = (a.wave_start[s + 1] - a.wave_start[s]) / a.Hkv;  // the pair's waves = its slots
    // slot of wave r of the pair (the decode kernel's interleave): r*pairs + pair
    // when every sequence has k waves per pair, else first(s) + r*Hkv + h
    const int w0 = a.k_uniform > 0 ? pair : a.wave_start[s] + h;
    const int slot_step = a.k_uniform > 0 ? a.n_seqs * a.Hkv : a.Hkv;
    const int nslot = k;
    const int64_t stride = (int64_t)slot_step * G * Dp;  // floats between the pair's consecutive slots
    const float *base = a.ws + ((int64_t)w0 * G + gg) * Dp;
    const int t = threadIdx.x, c = t % D, grp = t / D;
    float *const dst = a.out + ((int64_t)s * a.Hq + (int64_t)h * G + gg) * D + c;

    if (nslot <= 16) {
        // few slots (the usual case): one thread per channel loads the (m, l)
        // and O of every slot at once -- one round trip, no barriers
        if (grp > 0)
            return;  // whole waves: D is a multiple of 64
        const float r = nslot <= 8 ? merge_few<8>(base, stride, nslot, c, D) : merge_few<16>(base, stride, nslot, c, D);
        *dst = a.v_rotated ? rotate_back(r, c) : r;
        return;
    }

    if (nslot <= 16 * P && nslot <= (int)blockDim.x) {
        // up to 16 slots per group: thread t loads slot t's (m, l), and each
        // thread the O values of its group's slots grp, grp+P, ... -- all
        // loads issued together, one round trip; then the maximum, the
        // weights (through LDS) and the sums
        float mt = -INFINITY, lt = 0.0f;
        if (t < nslot) {
            mt = base[(int64_t)t * stride + D];
            lt = base[(int64_t)t * stride + D + 1];
        }
        float ov[16];
#pragma unroll
        for (int u = 0; u < 16; u++)
            ov[u] = base[(int64_t)min(grp + u * P, nslot - 1) * stride + c];
        const float M = block_reduce(mt, red, true);
        const float w = t < nslot ? __builtin_amdgcn_exp2f(mt - M) : 0.0f;
        if (t < nslot)
            wts[t] = w;
        const float L = block_reduce(lt * w, red, false);  // its barriers also publish wts
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < 16; u++)
            if (grp + u * P < nslot)
                acc += ov[u] * wts[grp + u * P];
        if (P > 1) {
            part[t] = acc;
            __syncthreads();
            if (grp == 0)
                for (int g2 = 1; g2 < P; g2++)
                    acc += part[g2 * D + c];
        }
        float r = acc / L;
        if (a.v_rotated && grp == 0)  // whole waves take this branch
            r = rotate_back(r, c);
        if (grp == 0)
            *dst = r;
        return;
    }

    float mx = -INFINITY;
    for (int j = t; j < nslot; j += blockDim.x)
        mx = fmaxf(mx, base[j * stride + D]);
    const float M = block_reduce(mx, red, true);

    float lsum = 0.0f, acc = 0.0f;
    for (int k0 = 0; k0 < nslot; k0 += MERGE_CHUNK) {
        const int chunk = min(MERGE_CHUNK, nslot - k0);
        __syncthreads();  // the previous chunk's weights are no longer read
        for (int j = t; j < chunk; j += blockDim.x) {
            const float *pk = base + (int64_t)(k0 + j) * stride;
            const float w = __builtin_amdgcn_exp2f(pk[D] - M);
            wts[j] = w;
            lsum += pk[D + 1] * w;
        }
        __syncthreads();
        const float *pc = base + (int64_t)k0 * stride + c;
        int j = grp;
        // batches of U independent loads in flight, U = 16, then 8, 4, 1
        auto batch = [&](auto u_c) {
            constexpr int U = decltype(u_c)::value;
            for (; j + (U - 1) * P < chunk; j += U * P) {
                float v[U];
#pragma unroll
                for (int u = 0; u < U; u++)
                    v[u] = pc[(int64_t)(j + u * P) * stride];
#pragma unroll
                for (int u = 0; u < U; u++)
                    acc += v[u] * wts[j + u * P];
            }
        };
        batch(std::integral_constant<int, 16>());
        batch(std::integral_constant<int, 8>());
        batch(std::integral_constant<int, 4>());
        batch(std::integral_constant<int, 1>());
    }
    const float L = block_reduce(lsum, red, false);
    if (P > 1) {
        part[t] = acc;
        __syncthreads();
        if (grp == 0)
            for (int g2 = 1; g2 < P; g2++)
                acc += part[g2 * D + c];
    }
    float r = acc / L;
    if (a.v_rotated && grp == 0)  // whole waves take this branch
        r = rotate_back(r, c);
    if (grp == 0)
        *dst = r;
}

template <int KT, int VT, int D>
hipError_t launch_dec(const DecodeArgs &a, hipStream_t st)
{
    dim3 grid((a.W + WAVES - 1) / WAVES);
    hipLaunchKernelGGL((decode_kernel<KT, VT, D>), grid, dim3(64 * WAVES), 0, st, a);
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

hipError_t launch_decode(int kt, int vt, int D, const DecodeArgs &a, const MergeArgs &m, int n_pairs, hipStream_t st)
{
    hipError_t e;
    switch (D) {
    case 64: e = launch_dec_d<64>(kt, vt, a, st); break;
    case 128: e = launch_dec_d<128>(kt, vt, a, st); break;
    case 256: e = launch_dec_d<256>(kt, vt, a, st); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess)
        return e;
    // merge groups: about 16 slots per group for the longest merge
    int k_max = 1;
    for (int q = 0; q < n_pairs / m.Hkv; q++)
        k_max = std::max(k_max, (m.wave_start[q + 1] - m.wave_start[q]) / m.Hkv);
    int P = 1;
    while (P * 2 * m.D <= MERGE_MAX_THREADS && P * 16 < k_max)
        P *= 2;
    hipLaunchKernelGGL(merge_kernel, dim3(n_pairs * m.G), dim3(P * m.D), 0, st, m);
    return hipGetLastError();
}

}  // namespace kvq
