// kvq_prefill.hip -- causal chunked prefill over the quantized cache.
//
// A chunk of n_tok new queries per sequence, already appended at positions
// p0 .. p0+n_tok-1, attends causally: query i sees cache positions 0 .. p0+i.
// The chunk is the micro-batch of the llama.cpp guide's batch-size section
// ("Batch-Groessen-Abstimmung", the -ub flag).  Flash attention as in that
// guide's "Flash Attention" section: tiled, online softmax, exact.
//
// Rows are (query token, head of the GQA group) pairs, so all heads that share
// a kv head share every K/V tile.  A workgroup owns PW waves x 16*RB rows of
// one (sequence, kv head) and walks the keys in steps of SUB 32-token tiles
// (the layout per head_dim and pair is below); each tile is copied once into
// LDS (the waves deal out the copy instructions), its quantized blocks are
// turned into MFMA operands once for the workgroup (the waves deal out those
// jobs too and write the operands back to LDS), and all waves read them.  The
// operands of step t+1 are built while step t is computed, one barrier per
// step, so that each wave's dequantization runs between its MFMAs.  Per wave
// and tile both contractions run on v_mfma_f32_16x16x32_f16, and every
// operand is shared by the wave's RB row blocks:
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

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), in order.
template <int N, class F>
__device__ inline __attribute__((always_inline)) void static_for_pf(F &&f)
{
    if constexpr (N > 0) {
        static_for_pf<N - 1>(f);
        f(std::integral_constant<int, N - 1>());
    }
}

// Rows, waves and step length of a workgroup.  Waves of two 16-row blocks
// fit in 256 registers, two waves per SIMD: at head_dim 128 eight of them
// in one workgroup per CU; at 64 eight (quantized values) or four in each of
// two workgroups per CU (binary16 values).  At 256 with a quantized half:
// eight waves of one row block, two waves per SIMD in one workgroup per CU
// (measured 36% faster for K8V4 than four waves of two blocks, whose
// 448-register waves ran alone on their SIMDs, the dequantization and the
// MFMAs largely one after the other).  f16/f16 at 256 keeps four waves of two
// blocks: with one block per wave it spilled.
// This file is compiled with the MFMA accumulators in VGPRs
// (-amdgpu-mfma-vgpr-form): the online-softmax rescale touches them with
// vector instructions, and with AGPR accumulators the compiler copied them
// between the two register files on every tile.
template <int KT, int VT, int D> struct Layout {
    static constexpr bool ONE = D == 256 && !(KT == KVQ_F16 && VT == KVQ_F16);
    // head_dim 64 with quantized values: eight waves, four tiles per step
    static constexpr bool W8_64 = D == 64 && VT != KVQ_F16;
    static constexpr int RB = ONE ? 1 : 2;  // 16-row blocks per wave
    static constexpr int PW = ONE || D == 128 || W8_64 ? 8 : 4;  // waves per workgroup
    static constexpr int WPE = D <= 128 || ONE ? 2 : 1;  // waves per SIMD the registers allow
    // 32-key tiles per step (one barrier, one softmax update).  A step's
    // barrier, copy waits, row maxima and rescale check cost the same
    // whatever its length, so longer steps spread them over more matrix work;
    // the step's raw tiles and operands must fit the LDS.  Head_dim 128: two
    // tiles, whose operands need the whole LDS (one workgroup of eight waves
    // per CU).  Head_dim 64: four tiles and eight waves where the values are
    // quantized, the same LDS; two tiles and two workgroups of four waves per
    // CU for binary16 values (with four tiles their raw operands spilled
    // registers).
    static constexpr int SUB = D == 64 ? (W8_64 ? 4 : 2) : D == 128 ? 2 : 1;
    static constexpr int LDS_KB = D == 64 && !W8_64 ? 80 : 160;  // LDS budget of a workgroup
};

__device__ inline half8 splat8(uint32_t pair) { return pack4(pair, pair, pair, pair); }

template <int KT, int VT, int D>
__global__ __launch_bounds__((64 * Layout<KT, VT, D>::PW)) __attribute__((amdgpu_waves_per_eu((Layout<KT, VT, D>::WPE)))) void prefill_kernel(const PrefillArgs a)
{
    using g = Geo<KT, VT, D>;
    constexpr int PW = Layout<KT, VT, D>::PW;
    constexpr int NB = g::NB, NCT = g::NCT;
    constexpr int RB = Layout<KT, VT, D>::RB;
    constexpr int SUB = Layout<KT, VT, D>::SUB, STEP = TILE * SUB;
    constexpr int ROWS_G = 16 * RB * PW;
    constexpr int VL = (VT == KVQ_Q4_0 || VT == KVQ_Q5_0 || VT == KVQ_TURBO3) ? NB : NCT;
    constexpr bool KQ = KT != KVQ_F16, VQ = VT != KVQ_F16;
    // raised issue priority from the dequantization through the scores (see
    // the score phase)
    constexpr bool PRIO_DQ = KQ || VQ;

    // Dequantized operands of the current tile, built once per workgroup:
    // K hi and lo per (tile u of the step, score tile T, block b), V (times
    // scale) per (u, block b, half hh); each set is one MFMA operand, 16 bytes
    // per lane, lane-major.
    constexpr int NKSET = KQ ? 2 * NB * SUB : 0, NVSET = VQ ? 2 * NB * SUB : 0;
    constexpr int DQ_KHI = 0, DQ_KLO = DQ_KHI + NKSET * 1024, DQ_V = DQ_KLO + NKSET * 1024;
    constexpr int DQ_BYTES = DQ_V + NVSET * 1024;
    // tile t's in dq0 (t even) or dq1 (t odd): two arrays, so that the
    // compiler sees that building one tile's operands does not touch the
    // other's, and may interleave the two.  The compiler lays the kernel's
    // LDS arrays out by decreasing alignment, then decreasing size; the
    // larger alignment puts the operand arrays below the raw steps whatever
    // their sizes, so that more of the operand reads (every wave, every
    // tile) sit within the 64 KiB a DS instruction's offset field reaches
    // from the lane's base address and need no address instruction of their
    // own.
    __shared__ __attribute__((aligned(DQ_BYTES > 0 ? 32 : 16))) uint8_t dq0[DQ_BYTES > 0 ? DQ_BYTES : 16];
    __shared__ __attribute__((aligned(DQ_BYTES > 0 ? 32 : 16))) uint8_t dq1[DQ_BYTES > 0 ? DQ_BYTES : 16];
    // raw steps (SUB tiles each, tile u at u * g::BYTES): step t in
    // lds[t % NRAW].  While t is computed, t+1 is being dequantized and the
    // copies of the later steps are in flight: t+2 with three buffers, t+2
    // and t+3 with four, which every pair gets where they fit beside the
    // operand arrays at the workgroups per CU the kernel is built for (two at
    // head_dim <= 128, one at 256)
    constexpr int LDS_WG = Layout<KT, VT, D>::LDS_KB * 1024;
    constexpr int NRAW = 4 * SUB * g::BYTES + 2 * (DQ_BYTES > 0 ? DQ_BYTES : 16) <= LDS_WG ? 4 : 3;
    __shared__ __attribute__((aligned(16))) uint8_t lds[NRAW][SUB * g::BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Binary16 keys in the eight-wave layouts (head_dim 128; head_dim 64 with
    // quantized values): only the first half of the waves raises its issue
    // priority in the phases below, so the two waves that share a SIMD (w and
    // w + 4) do not move through their matrix and vector phases in step
    // (1.5-2.7% faster for those pairs at head_dim 128, 3-4% at 64; with
    // quantized keys, whose dequantization already spreads the phases, it was
    // slower).
    const bool prio_w = !(KT == KVQ_F16 && (D == 128 || Layout<KT, VT, D>::W8_64)) || wave < PW / 2;
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

    const int ntile = (key_end + STEP - 1) / STEP;  // steps

    // ---- dequantization of step t (raw copy in lds[t % NRAW]) into dqt,
    // the operand array of its parity (dq0 or dq1).  The step's jobs are K
    // sets (u, T, b), then V blocks (u, b); this wave takes jobs wave,
    // wave + PW, ...  As 2*NB*SUB is a multiple of PW, the i-th job of every
    // wave is of the same kind: straight-line code with wave-uniform offsets.
    // MASK: the step may reach past key_end.
    static_assert(!KQ || (2 * NB * SUB) % PW == 0, "K jobs are dealt evenly");
    auto dequant = [&](auto mask_c, const int t, uint8_t *const dqt) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_c)::value;
        constexpr int NKJ = KQ ? 2 * NB * SUB : 0, NJOB = NKJ + (VQ ? NB * SUB : 0);
#pragma unroll
        for (int i = 0; i < (NJOB + PW - 1) / PW; i++) {
            const int job = wave + PW * i;
            if (PW * i < NKJ) {
                const int u = SUB == 1 ? 0 : job / (2 * NB), T = SUB == 1 ? job / NB : (job / NB) & 1;
                const int b = job - (job / NB) * NB;
                const uint8_t *buf = lds[t % NRAW] + u * g::BYTES;
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
                    ka = k_operand_q5(w, hw, 4 * j);
                }
                const uint16_t dbits = *reinterpret_cast<const uint16_t *>(buf + g::KS_OFF + (r * NB + b) * 2);
                const half8 dd = splat8(dbits * 0x00010001u);
                const half8 hi = ka * dd;
                const half8 lo = __builtin_elementwise_fma(ka, dd, -hi);
                *reinterpret_cast<half8 *>(dqt + DQ_KHI + (job * 64 + lane) * 16) = hi;
                *reinterpret_cast<half8 *>(dqt + DQ_KLO + (job * 64 + lane) * 16) = lo;
            } else if (VQ && (NJOB % PW == 0 || job < NJOB)) {  // waves < PW: only a ragged last round checks
                const int u = SUB == 1 ? 0 : (job - NKJ) / NB, b = job - NKJ - u * NB;
                const uint8_t *buf = lds[t % NRAW] + u * g::BYTES;
                const int tb = t * STEP + TILE * u;
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
                    *reinterpret_cast<half8 *>(dqt + DQ_V + ((2 * NB * u + 2 * b + hh) * 64 + lane) * 16) = va[hh] * dv;
            }
        }
    };

    // ---- one step's attention from its operands (dqt, and the raw tiles
    // for binary16 planes); DG: the step may hold keys past a row's
    // position (masking).  Key r of lane group j in tile u is
    // t * STEP + TILE * u + 8 j + r.
    auto compute = [&](auto diag_c, const int t, const uint8_t *const dqt) __attribute__((always_inline)) {
        constexpr bool DG = decltype(diag_c)::value;
        const uint8_t *buf = lds[t % NRAW];
        const int tb = t * STEP;
        // raw f16 operands (no dequantization) stay in the raw tiles.  With
        // two tiles per step they are read where they are used (read up
        // front, both tiles' operands would not fit the registers).
        constexpr bool LATE = SUB == 2;
        u32x4 kop[SUB][2][NB];
        u32x4 vop[SUB][VL];
        if (!KQ && !LATE) {
#pragma unroll
            for (int u = 0; u < SUB; u++)
#pragma unroll
                for (int T = 0; T < 2; T++)
#pragma unroll
                    for (int b = 0; b < NB; b++)
                        kop[u][T][b] = *reinterpret_cast<const u32x4 *>(buf + u * g::BYTES + k_rd[T][b]);
        }
        // keys at or past key_end in binary16 V tiles: values forced to +0
        uint32_t vkm[SUB][4];
        if (!VQ && LATE && DG) {
#pragma unroll
            for (int u = 0; u < SUB; u++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int k0 = tb + TILE * u + 8 * j + 2 * i;
                    vkm[u][i] = (k0 < key_end ? 0x0000FFFFu : 0u) | (k0 + 1 < key_end ? 0xFFFF0000u : 0u);
                }
        }
        if (!VQ && !LATE) {
#pragma unroll
            for (int u = 0; u < SUB; u++) {
#pragma unroll
                for (int i = 0; i < VL; i++)
                    vop[u][i] = *reinterpret_cast<const u32x4 *>(buf + u * g::BYTES + v_rd[i]);
                if (DG && tb + TILE * (u + 1) > key_end) {
                    uint32_t vk[4];
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int k0 = tb + TILE * u + 8 * j + 2 * i;
                        vk[i] = (k0 < key_end ? 0x0000FFFFu : 0u) | (k0 + 1 < key_end ? 0xFFFF0000u : 0u);
                    }
#pragma unroll
                    for (int i = 0; i < VL; i++)
                        vop[u][i] = u32x4{vop[u][i].x & vk[0], vop[u][i].y & vk[1], vop[u][i].z & vk[2], vop[u][i].w & vk[3]};
                }
            }
        }
        // ---- scores.  The two contraction phases raise the wave's issue
        // priority (s_setprio), so that while one wave of a SIMD streams its
        // MFMAs the other wave's softmax fills the vector slots between them.
        // The priority change is a scheduling boundary, so where the next
        // tile's dequantization is interleaved with the score MFMAs, the
        // raised span starts before that dequantization (body below): for
        // every pair that dequantizes a half (with two-tile steps, K4V4 and
        // q4_0/q5_0 4-6% faster, quantized keys with binary16 values 5-7%,
        // binary16 keys 0-3%)
        constexpr bool PRIO_QK = !KQ && !VQ;
        if (PRIO_QK)
            if (prio_w) __builtin_amdgcn_s_setprio(1);
        floatx4 sacc[RB][2 * SUB];  // score tile 2u + T
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
#pragma unroll
            for (int x = 0; x < 2 * SUB; x++)
                sacc[rb][x] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < SUB; u++)
#pragma unroll
            for (int T = 0; T < 2; T++)
#pragma unroll
                for (int b = 0; b < NB; b++) {
                    const int x = 2 * u + T;
                    if (KT == KVQ_F16) {
                        const u32x4 w = LATE ? *reinterpret_cast<const u32x4 *>(buf + u * g::BYTES + k_rd[T][b]) : kop[u][T][b];
                        const half8 ka = pack4(w.x, w.y, w.z, w.w);
#pragma unroll
                        for (int rb = 0; rb < RB; rb++)
                            sacc[rb][x] = mfma(ka, qb[rb][b], sacc[rb][x]);
                    } else {
                        const int set = (2 * u + T) * NB + b;
                        const half8 hi = *reinterpret_cast<const half8 *>(dqt + DQ_KHI + (set * 64 + lane) * 16);
                        const half8 lo = *reinterpret_cast<const half8 *>(dqt + DQ_KLO + (set * 64 + lane) * 16);
#pragma unroll
                        for (int rb = 0; rb < RB; rb++) {
                            sacc[rb][x] = mfma(hi, qb[rb][b], sacc[rb][x]);
                            sacc[rb][x] = mfma(lo, qb[rb][b], sacc[rb][x]);
                        }
                    }
                }

        if (PRIO_QK || PRIO_DQ)
            if (prio_w) __builtin_amdgcn_s_setprio(0);
        // ---- online softmax per row block; score x = 8u + r of a lane is key
        // tb + 32u + 8j + r
        constexpr int NS = 8 * SUB;
        half8 pb[RB][SUB];
        const bool diag = DG && tb + STEP - 1 > wave_first;  // some key of the step is past some row's position
#pragma unroll
        for (int rb = 0; rb < RB; rb++) {
            float sc[NS];
#pragma unroll
            for (int x = 0; x < NS; x++)
                sc[x] = sacc[rb][x >> 2][x & 3];
            if (diag) {
#pragma unroll
                for (int x = 0; x < NS; x++)
                    if (tb + TILE * (x >> 3) + 8 * j + (x & 7) > lim[rb])
                        sc[x] = -INFINITY;
            }
            float mt = max3(max3(sc[0], sc[1], sc[2]), max3(sc[3], sc[4], sc[5]), max3(sc[6], sc[7], sc[7]));
#pragma unroll
            for (int u = 1; u < SUB; u++) {
                const float *q = sc + 8 * u;
                mt = max3(mt, max3(max3(q[0], q[1], q[2]), max3(q[3], q[4], q[5]), q[6]), q[7]);
            }
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
            float p[NS];
#pragma unroll
            for (int x = 0; x < NS; x++)
                p[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[x], c2a, nm));
            if (diag) {
#pragma unroll
                for (int x = 0; x < NS; x++)
                    p[x] = (sc[x] == -INFINITY) ? 0.0f : p[x];
            }
#pragma unroll
            for (int u = 0; u < SUB; u++) {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    w[i] = h2_bits(__builtin_convertvector((float2v){p[8 * u + 2 * i], p[8 * u + 2 * i + 1]}, half2));
                pb[rb][u] = pack4(w[0], w[1], w[2], w[3]);
            }
        }

        // ---- O^T += V^T . P (at priority 2 above the score phase where two
        // workgroups share a CU: their waves are not in lockstep, and this
        // orders the three phases -- head_dim 64 with binary16 values,
        // f16/f16 10% faster; with one workgroup per CU it made no difference)
        if (prio_w) __builtin_amdgcn_s_setprio(Layout<KT, VT, D>::LDS_KB < 160 ? 2 : 1);
#pragma unroll
        for (int u = 0; u < SUB; u++)
#pragma unroll
            for (int b = 0; b < NB; b++) {
                half8 va[2];
                if (VQ) {
#pragma unroll
                    for (int hh = 0; hh < 2; hh++)
                        va[hh] = *reinterpret_cast<const half8 *>(dqt + DQ_V + ((2 * NB * u + 2 * b + hh) * 64 + lane) * 16);
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) {
                        u32x4 w;
                        if (LATE) {
                            w = *reinterpret_cast<const u32x4 *>(buf + u * g::BYTES + v_rd[2 * b + hh]);
                            if (DG)
                                w = u32x4{w.x & vkm[u][0], w.y & vkm[u][1], w.z & vkm[u][2], w.w & vkm[u][3]};
                        } else {
                            w = vop[u][2 * b + hh];
                        }
                        va[hh] = pack4(w.x, w.y, w.z, w.w);
                    }
                }
#pragma unroll
                for (int rb = 0; rb < RB; rb++) {
                    o[rb][2 * b] = mfma(va[0], pb[rb][u], o[rb][2 * b]);
                    o[rb][2 * b + 1] = mfma(va[1], pb[rb][u], o[rb][2 * b + 1]);
                }
            }
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
#pragma unroll
            for (int u = 0; u < SUB; u++)
                lacc[rb] = mfma(ones, pb[rb][u], lacc[rb]);
        if (prio_w) __builtin_amdgcn_s_setprio(0);
    };

    // ---- the step loop: one barrier per step.  At the barrier of step t,
    // step t+1's copy has landed (each wave waited for its share), step t's
    // operands are complete, and every wave is done with step t-1's operands
    // and with the raw buffer of step t-1.  Then: start the copy of step
    // t+NRAW-1 into that buffer, build step t+1's operands, and compute step
    // t -- the dequantization's vector instructions run beside the MFMAs.
    // dqw, dqr: the operand buffers of steps t+1 and t.  In the loops they
    // are the arrays themselves (pairs of steps per round), so that the
    // compiler may move step t's operand reads and MFMAs in between step
    // t+1's dequantization.
    // Copy of step t: instruction i of its tile u is issued by wave
    // (u * NDMA + i) % PW.  Vector-memory loads complete in issue order, so
    // waiting until at most this wave's share of one step is outstanding
    // means that the step before the last one issued has landed.
    constexpr int NDMA = g::NDMA, NDMA_S = SUB * NDMA;
    static_assert((NDMA_S + PW - 1) / PW < 64, "vmcnt holds 6 bits");
    auto issue_step = [&](const int t) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SUB; u++)
            issue_tile<KT, VT, D>(lds[t % NRAW] + u * g::BYTES, t * STEP + TILE * u, lane, doff, rs,
                                  u == 0 ? wave : (wave + PW - (u * NDMA) % PW) % PW, PW);
    };
    auto wait_share = [&]() __attribute__((always_inline)) {
        // wave w issues (NDMA_S + PW - 1 - w) / PW of a step's copy instructions
        static_for_pf<PW>([&](auto w) {
            constexpr int c = (NDMA_S + PW - 1 - decltype(w)::value) / PW;
            if (wave == decltype(w)::value)
                __builtin_amdgcn_s_waitcnt((c & 15) | ((c >> 4) << 14) | 0x70 | 0xF00);
        });
    };
    auto body = [&](auto diag_c, auto last2_c, const int t, uint8_t *const dqw, const uint8_t *const dqr) __attribute__((always_inline)) {
        constexpr bool LAST2 = decltype(last2_c)::value;  // t = ntile-2: no copy to start, dequant with mask
        if (NRAW >= 4 && !LAST2)
            wait_share();  // step t+1 landed; this wave's copies of step t+2 may still be in flight
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (NRAW >= 4) {
            if (!LAST2 && t + 3 < ntile)
                issue_step(t + 3);
        } else if (!LAST2) {
            issue_step(t + 2);
        }
        if (PRIO_DQ)
            if (prio_w) __builtin_amdgcn_s_setprio(1);  // through this dequantization and tile t's scores
        if (KQ || VQ)
            dequant(std::integral_constant<bool, LAST2>(), t + 1, dqw);
        compute(diag_c, t, dqr);
    };
    using F = std::integral_constant<bool, false>;
    using Tr = std::integral_constant<bool, true>;
    issue_step(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (ntile > 1)
        issue_step(1);
    if (NRAW >= 4 && ntile > 2)
        issue_step(2);
    if (KQ || VQ) {
        if (ntile > 1)
            dequant(F(), 0, dq0);
        else
            dequant(Tr(), 0, dq0);
    }
    // Steps before t_d lie entirely at or below every row position of this
    // wave and run without mask code.  Every wave still meets the same
    // barriers, those of ntile steps.
    const int t_d = min(ntile, (wave_first + 1) / STEP);
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
    // the last two steps (with the mask code, which checks at run time
    // whether a step needs it)
    if (ntile >= 2)
        body(Tr(), Tr(), ntile - 2, (ntile & 1) ? dq0 : dq1, (ntile & 1) ? dq1 : dq0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    compute(Tr(), ntile - 1, (ntile & 1) ? dq0 : dq1);

    // ---- turbo3 values: O was accumulated in the rotated basis; rotate each
    // 32-channel block of every row back
    if constexpr (VT == KVQ_TURBO3) {
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
            rotate_back_tiles<NCT>(o[rb], lane);
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
    constexpr int PW = Layout<KT, VT, D>::PW;
    constexpr int ROWS_G = 16 * Layout<KT, VT, D>::RB * PW;
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
