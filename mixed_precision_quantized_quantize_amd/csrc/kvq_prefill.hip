// kvq_prefill.hip -- causal chunked prefill over the quantized cache.
//
// A chunk of n_tok new queries per sequence, already appended at positions
// p0 .. p0+n_tok-1, attends causally: query i sees cache positions 0 .. p0+i.
// The chunk is the micro-batch of the llama.cpp guide's batch-size section
// ("Batch-Groessen-Abstimmung", the -ub flag).  Flash attention as in that
// guide's "Flash Attention" section: tiled, online softmax, exact.
//
// Rows are (query token, head of the GQA group) pairs, so all heads that share
// a kv head share every K/V tile.  A workgroup owns 4 waves x 16*RB rows of
// one (sequence, kv head) and walks the keys in 32-token tiles; each tile is
// copied once into LDS (the four waves deal out the copy instructions), its
// quantized blocks are turned into MFMA operands once for the workgroup (the
// four waves deal out those jobs too and write the operands back to LDS), and
// all four waves read them.  The operands of tile t+1 are built while tile t
// is computed, one barrier per tile, so that each wave's dequantization runs
// between its MFMAs.  Per wave and tile both contractions run on
// v_mfma_f32_16x16x32_f16, and every operand is shared by the wave's RB row
// blocks:
//   S^T[key][row]  = K[key][c] . Q^T[c][row]
//       A quantized K block enters as two binary16 operands hi + lo with
//       hi = fl16(code * d), lo = fl16(code * d - hi) (one fused multiply-add),
//       which together hold code * d exactly (the product has at most 8 + 11
//       significant bits), so the scale costs a second MFMA instead of a
//       vector multiply-add per (score, block);
//   O^T[c][row]   += V^T[c][key] . P[key][row]
//       with the V operand already multiplied by its block scale (binary16)
//       and P = binary16(p); one more MFMA against an all-ones operand sums
//       the same binary16 p into the softmax denominator.
// Online softmax in base 2: p = 2^(s*c2 - m), the subtraction folded into one
// fused multiply-add (a negative scale is moved onto Q, exactly).  Only tiles
// that reach past a row's own position are masked.
#include <type_traits>

#include "kvq_device.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

using namespace dev;

constexpr int PW = 4;  // waves per workgroup

// 16-row blocks per wave: two.  At head_dim <= 128 a wave then fits in 256
// registers and two workgroups share each CU (one wave's softmax then runs
// beside another's MFMAs); at 256 a wave takes up to 448 of 512 and the CU
// holds one workgroup, whose 128 rows still halve the dequantization per row
// (measured 35% faster than one row block).  This file is compiled with the
// MFMA accumulators in VGPRs (-amdgpu-mfma-vgpr-form): the online-softmax
// rescale touches them with vector instructions, and with AGPR accumulators
// the compiler copied them between the two register files on every tile.
template <int D> struct Rows { static constexpr int RB = 2; };

// max over the four lanes n, n+16, n+32, n+48 (the lane groups of one row)
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
// every MFMA result with an extra v_max_f32.  Scores are finite here, or
// -inf where masked (a masked key's garbage score is replaced before).
__device__ inline float max3(float a, float b, float c)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

__device__ inline half8 splat8(uint32_t pair) { return pack4(pair, pair, pair, pair); }

template <int KT, int VT, int D>
__global__ __launch_bounds__(64 * PW) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1))) void prefill_kernel(const PrefillArgs a)
{
    using g = Geo<KT, VT, D>;
    constexpr int NB = g::NB, NCT = g::NCT;
    constexpr int RB = Rows<D>::RB;
    constexpr int ROWS_G = 16 * RB * PW;
    constexpr int VL = (VT == KVQ_Q4_0 || VT == KVQ_Q5_0 || VT == KVQ_TURBO3) ? NB : NCT;
    constexpr bool KQ = KT != KVQ_F16, VQ = VT != KVQ_F16;
    // raised issue priority from the dequantization through the scores (see
    // the score phase)
    constexpr bool PRIO_DQ = (KT == KVQ_Q8_0 || KT == KVQ_Q5_0) && VQ;

    // Dequantized operands of the current tile, built once per workgroup:
    // K hi and lo per (score tile T, block b), V (times scale) per (block b,
    // half hh); each set is one MFMA operand, 16 bytes per lane, lane-major.
    constexpr int NKSET = KQ ? 2 * NB : 0, NVSET = VQ ? 2 * NB : 0;
    constexpr int DQ_KHI = 0, DQ_KLO = DQ_KHI + NKSET * 1024, DQ_V = DQ_KLO + NKSET * 1024;
    constexpr int DQ_BYTES = DQ_V + NVSET * 1024;
    // tile t's in dq0 (t even) or dq1 (t odd): two arrays, so that the
    // compiler sees that building one tile's operands does not touch the
    // other's, and may interleave the two
    __shared__ __attribute__((aligned(16))) uint8_t dq0[DQ_BYTES > 0 ? DQ_BYTES : 16];
    __shared__ __attribute__((aligned(16))) uint8_t dq1[DQ_BYTES > 0 ? DQ_BYTES : 16];
    // raw tiles: tile t in lds[t % NRAW].  While t is computed, t+1 is being
    // dequantized and the copies of the later tiles are in flight: t+2 with
    // three buffers, t+2 and t+3 with four, which every pair gets where they
    // fit beside the operand arrays at the workgroups per CU the kernel is
    // built for (two at head_dim <= 128, one at 256)
    constexpr int LDS_WG = (D <= 128 ? 80 : 160) * 1024;
    constexpr int NRAW = 4 * g::BYTES + 2 * (DQ_BYTES > 0 ? DQ_BYTES : 16) <= LDS_WG ? 4 : 3;
    __shared__ __attribute__((aligned(16))) uint8_t lds[NRAW][g::BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, j = lane >> 4;

    // Workgroups of one (sequence, kv head) are kept on one XCD (dispatch is
    // round-robin over the 8 XCDs) so that they share its L2 for K/V tiles.
    const int gx = gridDim.x, total = gx * gridDim.y * gridDim.z;
    int lin = blockIdx.x + gx * (blockIdx.y + gridDim.y * blockIdx.z);
    if (total % 8 == 0)
        lin = (lin % 8) * (total / 8) + lin / 8;
    const int qblk = lin % gx, h = (lin / gx) % gridDim.y, s = lin / (gx * gridDim.y);

    const int G = a.G, gsh = a.gp_log2;
    const int n_tok = a.n_tok, p0 = a.q_pos0[s];
    const int row0 = qblk * ROWS_G;
    const int tok_last = min(n_tok - 1, (row0 + ROWS_G - 1) >> gsh);
    const int key_end = p0 + tok_last + 1;  // keys [0, key_end) are visible to some row
    const int wrow0 = row0 + wave * 16 * RB;
    const int wave_first = p0 + min(wrow0 >> gsh, n_tok - 1);  // smallest last-visible key of the wave
    const int64_t pair = (int64_t)s * a.Hkv + h;
    const int64_t Tc = a.Tc;
    const float c2a = fabsf(a.c2);
    const bool neg = a.c2 < 0.0f;

    // this lane's row in each row block: (token, head g) = (gr >> gsh, gr & (Gp-1))
    int tok[RB], lim[RB];
    bool valid[RB];
    half8 qb[RB][NB];
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
        const int gr = wrow0 + rb * 16 + n;
        tok[rb] = gr >> gsh;
        const int gg = gr & ((1 << gsh) - 1);
        valid[rb] = gg < G && tok[rb] < n_tok;
        lim[rb] = min(p0 + tok[rb], key_end - 1);  // last visible key (rows past the chunk: padding)
        const _Float16 *qrow = reinterpret_cast<const _Float16 *>(a.q) +
                               (((int64_t)s * n_tok + min(tok[rb], n_tok - 1)) * a.Hq + (int64_t)h * G + min(gg, G - 1)) * D;
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const _Float16 v = qrow[32 * b + qk_chan<KT>(j, r)];
                qb[rb][b][r] = valid[rb] ? (neg ? -v : v) : (_Float16)0.0f;
            }
    }

    PairRsrc rs;
    rs.kc = make_rsrc(a.kc + pair * Tc * g::RK, Tc * g::RK);
    rs.vc = make_rsrc(a.vc + pair * Tc * g::RV, Tc * g::RV);
    if (KQ)
        rs.ks = make_rsrc(a.ks + pair * Tc * NB, Tc * NB * 2);
    if (VQ)
        rs.vs = make_rsrc(a.vs + pair * Tc * NB, Tc * NB * 2);
    if (KT == KVQ_Q5_0)
        rs.kh = make_rsrc(a.kqh + pair * Tc * NB, Tc * NB * 4);
    if (has_bit_words(VT))
        rs.vh = make_rsrc(a.vqh + pair * Tc * NB, Tc * NB * 4);
    DmaOffsets<KT, VT, D> doff;
    doff.init(lane);

    // LDS read offsets of the raw tile: K codes of score tile T (16 keys) and
    // block b; V codes as in decode
    int k_rd[2][NB];
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
    int v_rd[VL];
#pragma unroll
    for (int i = 0; i < VL; i++) {
        const int u = (VT == KVQ_TURBO3) ? 8 * i + (n & 7) : 16 * i + n;
        const int c = (VT == KVQ_F16) ? u : (u >> 1);
        const int within = (VT == KVQ_F16) ? 0 : 8 * (u & 1);
        v_rd[i] = g::V_OFF + (j * g::CPG + (c ^ vswz<VT, g::CPG>(j))) * 16 + within;
    }

    const half8 ones = splat8(0x3C003C00u);
    float m_run[RB];
    floatx4 o[RB][NCT], lacc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
        m_run[rb] = -INFINITY;
        lacc[rb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
            o[rb][ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const int ntile = (key_end + TILE - 1) / TILE;

    // ---- dequantization of tile t (raw copy in lds[t % NRAW]) into dqt,
    // the operand array of its parity (dq0 or dq1).  The tile's jobs are K sets (T, b), then V blocks b; this
    // wave takes jobs wave, wave + PW, ...  As 2*NB is a multiple of PW, the
    // i-th job of every wave is of the same kind: straight-line code with
    // wave-uniform offsets.  MASK: the tile may reach past key_end.
    static_assert(!KQ || (2 * NB) % PW == 0, "K jobs are dealt evenly");
    auto dequant = [&](auto mask_c, const int t, uint8_t *const dqt) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_c)::value;
        const uint8_t *buf = lds[t % NRAW];
        const int tb = t * TILE;
        constexpr int NKJ = KQ ? 2 * NB : 0, NJOB = NKJ + (VQ ? NB : 0);
#pragma unroll
        for (int i = 0; i < (NJOB + PW - 1) / PW; i++) {
            const int job = wave + PW * i;
            if (PW * i < NKJ) {
                const int T = job / NB, b = job - T * NB;
                const int r = 8 * (n >> 2) + 4 * T + (n & 3);  // this lane's key in the tile
                const int c = (KT == KVQ_Q8_0) ? 2 * b + (j >> 1) : b;
                const int within = (KT == KVQ_Q8_0) ? 8 * (j & 1) : 4 * j;
                const int krd = g::K_OFF + (r * g::CPR + (c ^ kswz<g::CPR>(r))) * 16 + within;
                half8 ka;
                if (KT == KVQ_Q8_0) {
                    const u32x2 w = *reinterpret_cast<const u32x2 *>(buf + krd);
                    ka = deq_q8(w.x, w.y);
                } else if (KT == KVQ_Q4_0) {
                    const uint32_t w = *reinterpret_cast<const uint32_t *>(buf + krd);
                    ka = k_operand<KVQ_Q4_0>(&w);
                } else {
                    const uint32_t w = *reinterpret_cast<const uint32_t *>(buf + krd);
                    const uint32_t hw = *reinterpret_cast<const uint32_t *>(buf + g::KH_OFF + (r * NB + b) * 4);
                    ka = k_operand_q5(w, hw >> (4 * j));
                }
                const uint16_t dbits = *reinterpret_cast<const uint16_t *>(buf + g::KS_OFF + (r * NB + b) * 2);
                const half8 dd = splat8(dbits * 0x00010001u);
                const half8 hi = ka * dd;
                const half8 lo = __builtin_elementwise_fma(ka, dd, -hi);
                *reinterpret_cast<half8 *>(dqt + DQ_KHI + (job * 64 + lane) * 16) = hi;
                *reinterpret_cast<half8 *>(dqt + DQ_KLO + (job * 64 + lane) * 16) = lo;
            } else if (VQ && (NJOB % PW == 0 || job < NJOB)) {  // waves < PW: only a ragged last round checks
                const int b = job - NKJ;
                // LDS offset of the codes a lane reads for operand u (as v_rd)
                auto vrd = [&](const int u_i) {
                    const int u = (VT == KVQ_TURBO3) ? 8 * u_i + (n & 7) : 16 * u_i + n;
                    return g::V_OFF + (j * g::CPG + ((u >> 1) ^ vswz<VT, g::CPG>(j))) * 16 + 8 * (u & 1);
                };
                u32x4 vsc = *reinterpret_cast<const u32x4 *>(buf + g::VS_OFF + (j * NB + b) * 16);
                // keys at or past key_end were never written for this chunk:
                // their scale bits may be anything, even NaN -> force zero
                if (MASK && tb + TILE > key_end) {
                    uint32_t vk[4];
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const int k0 = tb + 8 * j + 2 * q;
                        vk[q] = (k0 < key_end ? 0x0000FFFFu : 0u) | (k0 + 1 < key_end ? 0xFFFF0000u : 0u);
                    }
                    vsc = u32x4{vsc.x & vk[0], vsc.y & vk[1], vsc.z & vk[2], vsc.w & vk[3]};
                }
                half8 va[2];
                if (VT == KVQ_TURBO3) {
                    const u32x2 w = *reinterpret_cast<const u32x2 *>(buf + vrd(b));
                    const u32x4 *hp = reinterpret_cast<const u32x4 *>(buf + g::VH_OFF + (j * NB + b) * 32);
                    const u32x4 h0 = hp[0], h1 = hp[1];
                    const uint32_t h[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                    v_operand_tq3(w, h, n, va[0], va[1]);  // levels of the rotated values
                } else if (VT == KVQ_Q5_0) {
                    const u32x2 w = *reinterpret_cast<const u32x2 *>(buf + vrd(b));
                    const u32x4 *hp = reinterpret_cast<const u32x4 *>(buf + g::VH_OFF + (j * NB + b) * 32);
                    const u32x4 h0 = hp[0], h1 = hp[1];
                    const uint32_t h[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                    v_operand_q5(w, h, n, va[0], va[1]);
                } else if (VT == KVQ_Q4_0) {
                    const u32x2 w = *reinterpret_cast<const u32x2 *>(buf + vrd(b));
                    uint32_t l01, h01, l23, h23, l45, h45, l67, h67;
                    deq_q4_pair(__builtin_amdgcn_perm(w.x, w.x, 0x0C010C00u), l01, h01);
                    deq_q4_pair(__builtin_amdgcn_perm(w.x, w.x, 0x0C030C02u), l23, h23);
                    deq_q4_pair(__builtin_amdgcn_perm(w.y, w.y, 0x0C010C00u), l45, h45);
                    deq_q4_pair(__builtin_amdgcn_perm(w.y, w.y, 0x0C030C02u), l67, h67);
                    va[0] = pack4(l01, l23, l45, l67);
                    va[1] = pack4(h01, h23, h45, h67);
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) {
                        const u32x2 w = *reinterpret_cast<const u32x2 *>(buf + vrd(2 * b + hh));
                        va[hh] = deq_q8(w.x, w.y);
                    }
                }
                const half8 dv = pack4(vsc.x, vsc.y, vsc.z, vsc.w);  // scales of keys 0..7
#pragma unroll
                for (int hh = 0; hh < 2; hh++)
                    *reinterpret_cast<half8 *>(dqt + DQ_V + ((2 * b + hh) * 64 + lane) * 16) = va[hh] * dv;
            }
        }
    };

    // ---- one tile's attention from its operands (dqt, and the raw tile for
    // binary16 planes); DG: the tile may hold keys past a row's
    // position (masking)
    auto compute = [&](auto diag_c, const int t, const uint8_t *const dqt) __attribute__((always_inline)) {
        constexpr bool DG = decltype(diag_c)::value;
        const uint8_t *buf = lds[t % NRAW];
        const int tb = t * TILE;
        // raw f16 operands (no dequantization) stay in the raw tile
        u32x4 kop[2][NB];
        u32x4 vop[VL];
        if (!KQ) {
#pragma unroll
            for (int T = 0; T < 2; T++)
#pragma unroll
                for (int b = 0; b < NB; b++)
                    kop[T][b] = *reinterpret_cast<const u32x4 *>(buf + k_rd[T][b]);
        }
        if (!VQ) {
#pragma unroll
            for (int i = 0; i < VL; i++)
                vop[i] = *reinterpret_cast<const u32x4 *>(buf + v_rd[i]);
            if (DG && tb + TILE > key_end) {
                uint32_t vk[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int k0 = tb + 8 * j + 2 * i;
                    vk[i] = (k0 < key_end ? 0x0000FFFFu : 0u) | (k0 + 1 < key_end ? 0xFFFF0000u : 0u);
                }
#pragma unroll
                for (int i = 0; i < VL; i++)
                    vop[i] = u32x4{vop[i].x & vk[0], vop[i].y & vk[1], vop[i].z & vk[2], vop[i].w & vk[3]};
            }
        }
        // ---- scores.  The two contraction phases raise the wave's issue
        // priority (s_setprio), so that while one wave of a SIMD streams its
        // MFMAs the other wave's softmax fills the vector slots between them.
        // The priority change is a scheduling boundary, so where the next
        // tile's dequantization is interleaved with the score MFMAs, the
        // raised span starts before that dequantization (body below), and
        // only for 8- and 5-bit keys with quantized values (1-3% faster); for
        // the other pairs it measured no faster, or slower (f16/q4_0 +3%,
        // K4V4 +1%)
        constexpr bool PRIO_QK = !KQ && !VQ;
        if (PRIO_QK)
            __builtin_amdgcn_s_setprio(1);
        floatx4 sacc[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
            sacc[rb][0] = sacc[rb][1] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int T = 0; T < 2; T++)
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (KT == KVQ_F16) {
                    const half8 ka = pack4(kop[T][b].x, kop[T][b].y, kop[T][b].z, kop[T][b].w);
#pragma unroll
                    for (int rb = 0; rb < RB; rb++)
                        sacc[rb][T] = mfma(ka, qb[rb][b], sacc[rb][T]);
                } else {
                    const int set = T * NB + b;
                    const half8 hi = *reinterpret_cast<const half8 *>(dqt + DQ_KHI + (set * 64 + lane) * 16);
                    const half8 lo = *reinterpret_cast<const half8 *>(dqt + DQ_KLO + (set * 64 + lane) * 16);
#pragma unroll
                    for (int rb = 0; rb < RB; rb++) {
                        sacc[rb][T] = mfma(hi, qb[rb][b], sacc[rb][T]);
                        sacc[rb][T] = mfma(lo, qb[rb][b], sacc[rb][T]);
                    }
                }
            }

        if (PRIO_QK || PRIO_DQ)
            __builtin_amdgcn_s_setprio(0);
        // ---- online softmax per row block; key r of lane group j is tb+8j+r
        half8 pb[RB];
        const bool diag = DG && tb + TILE - 1 > wave_first;  // some key of the tile is past some row's position
#pragma unroll
        for (int rb = 0; rb < RB; rb++) {
            float sc[8];
#pragma unroll
            for (int r = 0; r < 8; r++)
                sc[r] = sacc[rb][r >> 2][r & 3];
            if (diag) {
#pragma unroll
                for (int r = 0; r < 8; r++)
                    if (tb + 8 * j + r > lim[rb])
                        sc[r] = -INFINITY;
            }
            float mt = max3(max3(sc[0], sc[1], sc[2]), max3(sc[3], sc[4], sc[5]), max3(sc[6], sc[7], sc[7]));
            mt = max_lane_groups(mt) * c2a;  // NaN only for a fully masked row at scale 0: no update
            if (__any(mt > m_run[rb])) {
                const float m_new = fmaxf(m_run[rb], mt);
                const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);  // 0 on the first tile
                lacc[rb] *= alpha;
#pragma unroll
                for (int ct = 0; ct < NCT; ct++)
                    o[rb][ct] *= alpha;
                m_run[rb] = m_new;
            }
            const float nm = -m_run[rb];
            float p[8];
#pragma unroll
            for (int r = 0; r < 8; r++)
                p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c2a, nm));
            if (diag) {
#pragma unroll
                for (int r = 0; r < 8; r++)
                    p[r] = (sc[r] == -INFINITY) ? 0.0f : p[r];
            }
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                w[i] = h2_bits(__builtin_convertvector((float2v){p[2 * i], p[2 * i + 1]}, half2));
            pb[rb] = pack4(w[0], w[1], w[2], w[3]);
        }

        // ---- O^T += V^T . P
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int b = 0; b < NB; b++) {
            half8 va[2];
            if (VQ) {
#pragma unroll
                for (int hh = 0; hh < 2; hh++)
                    va[hh] = *reinterpret_cast<const half8 *>(dqt + DQ_V + ((2 * b + hh) * 64 + lane) * 16);
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    const u32x4 w = vop[2 * b + hh];
                    va[hh] = pack4(w.x, w.y, w.z, w.w);
                }
            }
#pragma unroll
            for (int rb = 0; rb < RB; rb++) {
                o[rb][2 * b] = mfma(va[0], pb[rb], o[rb][2 * b]);
                o[rb][2 * b + 1] = mfma(va[1], pb[rb], o[rb][2 * b + 1]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
            lacc[rb] = mfma(ones, pb[rb], lacc[rb]);
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- the tile loop: one barrier per tile.  At the barrier of tile t,
    // tile t+1's copy has landed (each wave waited for its share), tile t's
    // operands are complete, and every wave is done with tile t-1's operands
    // and with the raw buffer of tile t-1.  Then: start the copy of tile
    // t+NRAW-1 into that buffer, build tile t+1's operands, and compute tile
    // t -- the dequantization's vector instructions run beside the MFMAs.
    // dqw, dqr: the operand buffers of tiles t+1 and t.  In the loops they
    // are the arrays themselves (pairs of tiles per round), so that the
    // compiler may move tile t's operand reads and MFMAs in between tile
    // t+1's dequantization.
    // Wait until this wave's copies of the tile before the last one issued
    // have completed: instruction i of a tile's copy is issued by wave
    // i % PW, and vector-memory loads complete in issue order, so at most
    // this wave's share of one tile may remain outstanding.
    constexpr int NDMA = g::NDMA;
    static_assert(PW == 4 && (NDMA + 3) / 4 < 64, "vmcnt holds 6 bits");
    auto wait_share = [&]() __attribute__((always_inline)) {
        constexpr int c0 = (NDMA + 3) / 4, c1 = (NDMA + 2) / 4, c2 = (NDMA + 1) / 4, c3 = NDMA / 4;
        switch (wave) {
        case 0: __builtin_amdgcn_s_waitcnt((c0 & 15) | ((c0 >> 4) << 14) | 0x70 | 0xF00); break;
        case 1: __builtin_amdgcn_s_waitcnt((c1 & 15) | ((c1 >> 4) << 14) | 0x70 | 0xF00); break;
        case 2: __builtin_amdgcn_s_waitcnt((c2 & 15) | ((c2 >> 4) << 14) | 0x70 | 0xF00); break;
        default: __builtin_amdgcn_s_waitcnt((c3 & 15) | ((c3 >> 4) << 14) | 0x70 | 0xF00); break;
        }
    };
    auto body = [&](auto diag_c, auto last2_c, const int t, uint8_t *const dqw, const uint8_t *const dqr) __attribute__((always_inline)) {
        constexpr bool LAST2 = decltype(last2_c)::value;  // t = ntile-2: no copy to start, dequant with mask
        if (NRAW >= 4 && !LAST2)
            wait_share();  // tile t+1 landed; this wave's copies of tile t+2 may still be in flight
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (NRAW >= 4) {
            if (!LAST2 && t + 3 < ntile)
                issue_tile<KT, VT, D>(lds[(t + 3) % NRAW], (t + 3) * TILE, lane, doff, rs, wave, PW);
        } else if (!LAST2) {
            issue_tile<KT, VT, D>(lds[(t + 2) % NRAW], (t + 2) * TILE, lane, doff, rs, wave, PW);
        }
        if (PRIO_DQ)
            __builtin_amdgcn_s_setprio(1);  // through this dequantization and tile t's scores
        if (KQ || VQ)
            dequant(std::integral_constant<bool, LAST2>(), t + 1, dqw);
        compute(diag_c, t, dqr);
    };
    using F = std::integral_constant<bool, false>;
    using Tr = std::integral_constant<bool, true>;
    issue_tile<KT, VT, D>(lds[0], 0, lane, doff, rs, wave, PW);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (ntile > 1)
        issue_tile<KT, VT, D>(lds[1], TILE, lane, doff, rs, wave, PW);
    if (NRAW >= 4 && ntile > 2)
        issue_tile<KT, VT, D>(lds[2 % NRAW], 2 * TILE, lane, doff, rs, wave, PW);
    if (KQ || VQ) {
        if (ntile > 1)
            dequant(F(), 0, dq0);
        else
            dequant(Tr(), 0, dq0);
    }
    // Tiles before t_d lie entirely at or below every row position of this
    // wave and run without mask code.  Every wave still meets the same
    // barriers, those of ntile tiles.
    const int t_d = min(ntile, (wave_first + 1) / TILE);
    const int t_a = min(t_d, ntile - 2);
    int t = 0;
    for (; t + 2 <= t_a; t += 2) {
        body(F(), F(), t, dq1, dq0);
        body(F(), F(), t + 1, dq0, dq1);
    }
    if (t < t_a) {  // t even
        body(F(), F(), t, dq1, dq0);
        t++;
    }
    if (t < ntile - 2 && (t & 1)) {
        body(Tr(), F(), t, dq0, dq1);
        t++;
    }
    for (; t + 2 <= ntile - 2; t += 2) {
        body(Tr(), F(), t, dq1, dq0);
        body(Tr(), F(), t + 1, dq0, dq1);
    }
    if (t < ntile - 2) {  // t even
        body(Tr(), F(), t, dq1, dq0);
        t++;
    }
    // the last two tiles (with the mask code, which checks at run time
    // whether a tile needs it)
    if (ntile >= 2)
        body(Tr(), Tr(), ntile - 2, (ntile & 1) ? dq0 : dq1, (ntile & 1) ? dq1 : dq0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    compute(Tr(), ntile - 1, (ntile & 1) ? dq0 : dq1);

    // ---- turbo3 values: O was accumulated in the rotated basis; rotate each
    // 32-channel block back, x = s.(H y)/32.  Channel 32b + e of this lane's
    // row sits at e = 16(ct - 2b) + 4j + i: butterflies of span 1, 2 over i,
    // 4, 8 over the lane groups j (lanes 16 and 32 apart), 16 over ct.
    if constexpr (VT == KVQ_TURBO3) {
#pragma unroll
        for (int rb = 0; rb < RB; rb++) {
#pragma unroll
            for (int ct = 0; ct < NCT; ct++) {
                floatx4 &v = o[rb][ct];
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
            for (int b = 0; b < NB; b++) {
                const floatx4 lo = o[rb][2 * b], hi = o[rb][2 * b + 1];
                o[rb][2 * b] = lo + hi;
                o[rb][2 * b + 1] = lo - hi;
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int e = 16 * (ct & 1) + 4 * j + i;
                    o[rb][ct][i] *= ((TQ3_SIGNS >> e) & 1u) ? -0.03125f : 0.03125f;
                }
        }
    }

    // ---- normalize and write this lane's rows: channels 16ct + 4j + i
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
        if (valid[rb]) {
            const int gg = (wrow0 + rb * 16 + n) & ((1 << gsh) - 1);
            float *dst = a.out + (((int64_t)s * n_tok + tok[rb]) * a.Hq + (int64_t)h * G + gg) * D;
            const float inv = 1.0f / lacc[rb][0];
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
                *reinterpret_cast<floatx4 *>(dst + 16 * ct + 4 * j) = o[rb][ct] * inv;
        }
    }
}

template <int KT, int VT, int D>
hipError_t launch_pf(const PrefillArgs &a, hipStream_t st)
{
    constexpr int ROWS_G = 16 * Rows<D>::RB * PW;
    const int rows = a.n_tok << a.gp_log2;
    dim3 grid((rows + ROWS_G - 1) / ROWS_G, a.Hkv, a.n_seqs);
    hipLaunchKernelGGL((prefill_kernel<KT, VT, D>), grid, dim3(64 * PW), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_pf_d(int kt, int vt, const PrefillArgs &a, hipStream_t st)
{
#define KVQ_P(K, V) \
    if (kt == K && vt == V) return launch_pf<K, V, D>(a, st);
    KVQ_FOR_EACH_TYPE_PAIR(KVQ_P)
#undef KVQ_P
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(int kt, int vt, int D, const PrefillArgs &a, hipStream_t st)
{
    switch (D) {
    case 64: return launch_pf_d<64>(kt, vt, a, st);
    case 128: return launch_pf_d<128>(kt, vt, a, st);
    case 256: return launch_pf_d<256>(kt, vt, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
