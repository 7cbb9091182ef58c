// kvq_prefill.hip -- causal chunked prefill over the quantized cache.
//
// A chunk of n_tok new queries per sequence (the micro-batch of the llama.cpp
// guide's "Batch-Groessen-Abstimmung"), already appended at positions
// p0 .. p0+n_tok-1, attends causally: query i sees cache positions
// 0 .. p0+i.  The chunk is the micro-batch of the llama.cpp guide's
// batch-size section ("Batch-Groessen-Abstimmung", the -ub flag).  Flash
// attention as in that guide's "Flash Attention" section: tiled, online
// softmax, exact.
//
// Rows are (query token, head of the GQA group) pairs, so all heads that share
// a kv head share every K/V tile.  A workgroup owns 128 rows (4 waves x 32)
// of one (sequence, kv head) and walks the keys in 32-token tiles; each tile
// is copied once into LDS (the four waves deal out the copy instructions) and
// read by all four waves.  Per wave and tile, both contractions run on
// v_mfma_f32_16x16x32_f16 exactly as in decode:
//   S^T[key][row]  = K[key][c] . Q^T[c][row]   (raw codes, K scale per
//                                                 (key, block) after the MFMA)
//   O^T[c][row]   += V^T[c][key] . P'[key][row] (P' = binary16(p) * V scale)
// with the K and V operands unpacked once and shared by the wave's row
// blocks.  Only tiles that reach past a row's own position are masked.
#include "kvq_device.h"

namespace kvq {
namespace {

using namespace dev;

constexpr int PW = 4;  // waves per workgroup

template <int D> struct Rows { static constexpr int RB = (D == 256) ? 1 : 2; };  // 16-row blocks per wave

template <int KT, int VT, int D>
__global__ __launch_bounds__(64 * PW) void prefill_kernel(const PrefillArgs a)
{
    using g = Geo<KT, VT, D>;
    constexpr int NB = g::NB, NCT = g::NCT;
    constexpr int RB = Rows<D>::RB;
    constexpr int ROWS_G = 16 * RB * PW;
    constexpr int VL = (VT == KVQ_Q4_0) ? NB : NCT;

    __shared__ __attribute__((aligned(16))) uint8_t lds[2][g::BYTES];

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
    const int tok_first = row0 >> gsh;
    const int tok_last = min(n_tok - 1, (row0 + ROWS_G - 1) >> gsh);
    const int key_end = p0 + tok_last + 1;  // keys [0, key_end) are visible to some row
    const int64_t pair = (int64_t)s * a.Hkv + h;
    const int64_t Tc = a.Tc;

    // this lane's row in each row block: (token, head g) = (gr >> gsh, gr & (Gp-1))
    int tok[RB], lim[RB];
    bool valid[RB];
    half8 qb[RB][NB];
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
        const int gr = row0 + wave * 16 * RB + rb * 16 + n;
        tok[rb] = gr >> gsh;
        const int gg = gr & ((1 << gsh) - 1);
        valid[rb] = gg < G && tok[rb] < n_tok;
        lim[rb] = min(p0 + tok[rb], key_end - 1);  // last visible key (rows past the chunk: padding)
        const _Float16 *qrow = reinterpret_cast<const _Float16 *>(a.q) +
                               (((int64_t)s * n_tok + min(tok[rb], n_tok - 1)) * a.Hq + (int64_t)h * G + min(gg, G - 1)) * D;
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int r = 0; r < 8; r++)
                qb[rb][b][r] = valid[rb] ? qrow[32 * b + qk_chan<KT>(j, r)] : (_Float16)0.0f;
    }

    PairRsrc rs;
    rs.kc = make_rsrc(a.kc + pair * Tc * g::RK, Tc * g::RK);
    rs.vc = make_rsrc(a.vc + pair * Tc * g::RV, Tc * g::RV);
    if (KT != KVQ_F16)
        rs.ks = make_rsrc(a.ks + pair * Tc * NB, Tc * NB * 2);
    if (VT != KVQ_F16)
        rs.vs = make_rsrc(a.vs + pair * Tc * NB, Tc * NB * 2);
    DmaOffsets<KT, VT, D> doff;
    doff.init(lane);

    int k_rd[2][NB];
#pragma unroll
    for (int T = 0; T < 2; T++) {
        const int r = 8 * (n >> 2) + 4 * T + (n & 3);
#pragma unroll
        for (int b = 0; b < NB; b++) {
            int c, within;
            if (KT == KVQ_Q8_0) c = 2 * b + (j >> 1), within = 8 * (j & 1);
            else if (KT == KVQ_Q4_0) c = b, within = 4 * j;
            else c = 4 * b + j, within = 0;
            k_rd[T][b] = g::K_OFF + (r * g::CPR + (c ^ kswz<g::CPR>(r))) * 16 + within;
        }
    }
    int v_rd[VL];
#pragma unroll
    for (int i = 0; i < VL; i++) {
        const int u = 16 * i + n;
        const int c = (VT == KVQ_F16) ? u : (u >> 1);
        const int within = (VT == KVQ_F16) ? 0 : 8 * (u & 1);
        v_rd[i] = g::V_OFF + (j * g::CPG + (c ^ vswz<VT, g::CPG>(j))) * 16 + within;
    }

    const int bp16 = (lane ^ 16) << 2, bp32 = (lane ^ 32) << 2;
    const float c2 = a.c2;
    float m_run[RB], l_run[RB];
    floatx4 o[RB][NCT];
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.0f;
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
            o[rb][ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const int ntile = (key_end + TILE - 1) / TILE;
    issue_tile<KT, VT, D>(lds[0], 0, lane, doff, rs, wave, PW);
    for (int t = 0; t < ntile; t++) {
        const uint8_t *buf = lds[t & 1];
        const int tb = t * TILE;
        // every wave's share of this tile has landed before anyone reads it
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        // ---- operands of the tile into registers
        u32x4 kop[2][NB];
        uint32_t ksc[4 * NB];
        u32x4 vop[VL];
        u32x4 vsc[NB];
#pragma unroll
        for (int T = 0; T < 2; T++)
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (KT == KVQ_F16) {
                    kop[T][b] = *reinterpret_cast<const u32x4 *>(buf + k_rd[T][b]);
                } else if (KT == KVQ_Q8_0) {
                    const u32x2 w = *reinterpret_cast<const u32x2 *>(buf + k_rd[T][b]);
                    kop[T][b] = u32x4{w.x, w.y, 0u, 0u};
                } else {
                    kop[T][b] = u32x4{*reinterpret_cast<const uint32_t *>(buf + k_rd[T][b]), 0u, 0u, 0u};
                }
            }
        if (KT != KVQ_F16) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(buf + g::KS_OFF + 16 * NB * j);
#pragma unroll
            for (int i = 0; i < NB; i++) {
                const u32x4 w = p[i];
                ksc[4 * i] = w.x, ksc[4 * i + 1] = w.y, ksc[4 * i + 2] = w.z, ksc[4 * i + 3] = w.w;
            }
        }
#pragma unroll
        for (int i = 0; i < VL; i++) {
            if (VT == KVQ_F16) {
                vop[i] = *reinterpret_cast<const u32x4 *>(buf + v_rd[i]);
            } else {
                const u32x2 w = *reinterpret_cast<const u32x2 *>(buf + v_rd[i]);
                vop[i] = u32x4{w.x, w.y, 0u, 0u};
            }
        }
        if (VT != KVQ_F16) {
#pragma unroll
            for (int b = 0; b < NB; b++)
                vsc[b] = *reinterpret_cast<const u32x4 *>(buf + g::VS_OFF + (j * NB + b) * 16);
        }
        // keys at or past key_end were never written for this chunk: their
        // value bits (and V scales) may be anything, even NaN -> force zero
        if (tb + TILE > key_end) {
            uint32_t vk[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int k0 = tb + 8 * j + 2 * i;
                vk[i] = (k0 < key_end ? 0x0000FFFFu : 0u) | (k0 + 1 < key_end ? 0xFFFF0000u : 0u);
            }
            if (VT == KVQ_F16) {
#pragma unroll
                for (int i = 0; i < VL; i++)
                    vop[i] = u32x4{vop[i].x & vk[0], vop[i].y & vk[1], vop[i].z & vk[2], vop[i].w & vk[3]};
            } else {
#pragma unroll
                for (int b = 0; b < NB; b++)
                    vsc[b] = u32x4{vsc[b].x & vk[0], vsc[b].y & vk[1], vsc[b].z & vk[2], vsc[b].w & vk[3]};
            }
        }
        // start the next tile's copy into the other buffer (its last readers
        // finished before this iteration's barrier)
        if (t + 1 < ntile)
            issue_tile<KT, VT, D>(lds[(t + 1) & 1], tb + TILE, lane, doff, rs, wave, PW);

        // ---- scores for every row block (K operand unpacked once)
        floatx4 sacc[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
            sacc[rb][0] = sacc[rb][1] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int T = 0; T < 2; T++)
#pragma unroll
            for (int b = 0; b < NB; b++) {
                half8 ka;
                if (KT == KVQ_F16) {
                    ka = pack4(kop[T][b].x, kop[T][b].y, kop[T][b].z, kop[T][b].w);
                } else if (KT == KVQ_Q8_0) {
                    ka = deq_q8(kop[T][b].x, kop[T][b].y);
                } else {
                    const uint32_t w = kop[T][b].x;
                    ka = k_operand<KVQ_Q4_0>(&w);
                }
#pragma unroll
                for (int rb = 0; rb < RB; rb++) {
                    if (KT == KVQ_F16) {
                        sacc[rb][T] = mfma(ka, qb[rb][b], sacc[rb][T]);
                    } else {
                        const floatx4 c = mfma(ka, qb[rb][b], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            sacc[rb][T][i] = __builtin_fmaf(half_at(ksc, (4 * T + i) * NB + b), c[i], sacc[rb][T][i]);
                    }
                }
            }

        // ---- online softmax per row block; key r of lane group j is tb+8j+r
        uint32_t p16[RB][4];
        const bool diag = tb + TILE - 1 > p0 + tok_first;  // some key is past some row's position
#pragma unroll
        for (int rb = 0; rb < RB; rb++) {
            float x[8];
#pragma unroll
            for (int r = 0; r < 8; r++)
                x[r] = sacc[rb][r >> 2][r & 3] * c2;
            if (diag) {
#pragma unroll
                for (int r = 0; r < 8; r++)
                    if (tb + 8 * j + r > lim[rb])
                        x[r] = -INFINITY;
            }
            float mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            mt = fmaxf(mt, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp16, __builtin_bit_cast(int, mt))));
            mt = fmaxf(mt, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp32, __builtin_bit_cast(int, mt))));
            // key 0 is visible to every row, so m_run is finite after the
            // first tile; a fully masked row of a later tile has mt = -inf
            if (__any(mt > m_run[rb])) {
                const float m_new = fmaxf(m_run[rb], mt);
                const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);  // 0 on the first tile
                l_run[rb] *= alpha;
#pragma unroll
                for (int ct = 0; ct < NCT; ct++)
                    o[rb][ct] *= alpha;
                m_run[rb] = m_new;
            }
            float p[8];
#pragma unroll
            for (int r = 0; r < 8; r++) {
                p[r] = __builtin_amdgcn_exp2f(x[r] - m_run[rb]);
                l_run[rb] += p[r];
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
                p16[rb][i] = h2_bits(__builtin_convertvector((float2v){p[2 * i], p[2 * i + 1]}, half2));
        }

        // ---- O^T += V^T . P' (V operand unpacked once per block)
#pragma unroll
        for (int b = 0; b < NB; b++) {
            half8 va[2];
            if (VT == KVQ_Q4_0) {
                const u32x4 w = vop[b];
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
                    const u32x4 w = vop[2 * b + hh];
                    va[hh] = (VT == KVQ_F16) ? pack4(w.x, w.y, w.z, w.w) : deq_q8(w.x, w.y);
                }
            }
#pragma unroll
            for (int rb = 0; rb < RB; rb++) {
                half8 pb;
                if (VT == KVQ_F16) {
                    pb = pack4(p16[rb][0], p16[rb][1], p16[rb][2], p16[rb][3]);
                } else {
                    pb = pack4(h2_bits(bits_h2(p16[rb][0]) * bits_h2(vsc[b].x)),
                               h2_bits(bits_h2(p16[rb][1]) * bits_h2(vsc[b].y)),
                               h2_bits(bits_h2(p16[rb][2]) * bits_h2(vsc[b].z)),
                               h2_bits(bits_h2(p16[rb][3]) * bits_h2(vsc[b].w)));
                }
                o[rb][2 * b] = mfma(va[0], pb, o[rb][2 * b]);
                o[rb][2 * b + 1] = mfma(va[1], pb, o[rb][2 * b + 1]);
            }
        }
    }

    // ---- normalize and write this lane's rows: channels 16ct + 4j + i
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
        float l = l_run[rb] + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp16, __builtin_bit_cast(int, l_run[rb])));
        l += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp32, __builtin_bit_cast(int, l)));
        if (valid[rb]) {
            const int gg = (row0 + wave * 16 * RB + rb * 16 + n) & ((1 << gsh) - 1);
            float *dst = a.out + (((int64_t)s * n_tok + tok[rb]) * a.Hq + (int64_t)h * G + gg) * D;
            const float inv = 1.0f / l;
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
    KVQ_P(KVQ_F16, KVQ_F16) KVQ_P(KVQ_F16, KVQ_Q8_0) KVQ_P(KVQ_F16, KVQ_Q4_0)
    KVQ_P(KVQ_Q8_0, KVQ_F16) KVQ_P(KVQ_Q8_0, KVQ_Q8_0) KVQ_P(KVQ_Q8_0, KVQ_Q4_0)
    KVQ_P(KVQ_Q4_0, KVQ_F16) KVQ_P(KVQ_Q4_0, KVQ_Q8_0) KVQ_P(KVQ_Q4_0, KVQ_Q4_0)
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
