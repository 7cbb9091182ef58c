// kvq_decode.hip -- split-K flash decode over the quantized cache with the
// log-sum-exp merge of the split partials folded into the same launch.
//
// Flash attention in the sense of the llama.cpp guide's "Flash Attention"
// section (tiled, the score matrix never materialized, exactly softmax
// attention), reading the quantized blocks directly -- the KVSplit page's
// discussion expects the gain "integrated directly into FlashAttention", and
// the llama.cpp issue shows a quantized V cache is only usable that way.
//
// One workgroup = (split of the context, kv head, sequence), four waves.
// Each wave walks 32-token tiles of its split and serves the whole GQA group
// (up to 16 query heads) of its kv head with two matrix-core contractions
// per tile, both v_mfma_f32_16x16x32_f16:
//   S^T[token][head] = K[token][c] . Q^T[c][head]  -- one MFMA per 16 tokens
//       and 32-channel block; the raw codes are exact in binary16 and the
//       block's K scale multiplies the MFMA result per token;
//   O^T[chan][head] += V^T[chan][token] . P'[token][head]  -- one MFMA per 16
//       channels and 32 tokens; P' = binary16(p) * V scale of (token, block).
// The score layout of the first product is exactly the operand layout of the
// second, so probabilities never leave registers.  The V plane stores 8
// tokens interleaved, so a lane's P.V operand (8 tokens of one channel) is
// one 8- or 16-byte load.  Online softmax runs in base 2 (scores times
// scale*log2 e).  The next tile's codes and scales are loaded while the
// current one is computed.  The four waves' (m, l, O) merge in LDS; each
// workgroup writes one partial per query head, and the last workgroup of a
// (sequence, kv head) -- found with a device-scope counter -- merges all the
// partials and writes the normalized output.
#include "kvq_device.h"

namespace kvq {
namespace {

using namespace dev;

template <int KT, int VT, int D>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 3 : 1))) void decode_kernel(const DecodeArgs a)
{
    using g = Geo<KT, VT, D>;
    constexpr int NB = g::NB, NCT = g::NCT;

    __shared__ __attribute__((aligned(16))) uint8_t lds_a[g::LDS_A];
    __shared__ float sm_m[WAVES][16];
    __shared__ float sm_l[WAVES][16];
    __shared__ int sm_last;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
    const int n = lane & 15, j = lane >> 4;
    const int split = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int ctx = a.ctx_len[s];
    const int t_begin = split * a.tps;
    if (t_begin >= ctx)
        return;  // holds no tokens: not counted by the merge
    const int t_end = min(t_begin + a.tps, ctx);
    const int nsp = (ctx + a.tps - 1) / a.tps;
    const int G = a.G;
    const int64_t pair = (int64_t)s * a.Hkv + h;
    const int64_t Tc = a.Tc;

    // Q^T operand: lane (n = head, j) holds 8 channels of each block.
    half8 qb[NB];
    {
        const _Float16 *qrow =
            reinterpret_cast<const _Float16 *>(a.q) + ((int64_t)s * a.Hq + (int64_t)h * G + min(n, G - 1)) * D;
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int r = 0; r < 8; r++)
                qb[b][r] = (n < G) ? qrow[32 * b + qk_chan<KT>(j, r)] : (_Float16)0.0f;
    }

    PairRsrc rs;
    rs.kc = make_rsrc(a.kc + pair * Tc * g::RK, Tc * g::RK);
    rs.vc = make_rsrc(a.vc + pair * Tc * g::RV, Tc * g::RV);
    if (KT != KVQ_F16)
        rs.ks = make_rsrc(a.ks + pair * Tc * NB, Tc * NB * 2);
    if (VT != KVQ_F16)
        rs.vs = make_rsrc(a.vs + pair * Tc * NB, Tc * NB * 2);
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
            else if (KT == KVQ_Q4_0) c = b, within = 4 * j;
            else c = 4 * b + j, within = 0;
            k_rd[T][b] = g::K_OFF + (r * g::CPR + (c ^ kswz<g::CPR>(r))) * 16 + within;
        }
    }
    constexpr int VL = (VT == KVQ_Q4_0) ? NB : NCT;  // V operand reads per tile
    int v_rd[VL];
#pragma unroll
    for (int i = 0; i < VL; i++) {
        const int u = 16 * i + n;  // q4_0: byte n of block i; else channel 16i+n
        const int c = (VT == KVQ_F16) ? u : (u >> 1);
        const int within = (VT == KVQ_F16) ? 0 : 8 * (u & 1);
        v_rd[i] = g::V_OFF + (j * g::CPG + (c ^ vswz<VT, g::CPG>(j))) * 16 + within;
    }

    const int bp16 = (lane ^ 16) << 2, bp32 = (lane ^ 32) << 2;  // ds_bpermute byte addresses
    float m_run = -INFINITY;  // running max (base 2) of head n, equal in the 4 lane groups
    float l_run = 0.0f;       // this lane's share of the running sum
    floatx4 o[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ct++)
        o[ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // The operands of one tile, read from its LDS copy into registers.
    struct Ops {
        u32x4 k[2][NB];                 // K codes per S-tile and block (words used by the type)
        uint32_t ks[4 * NB];            // K scales: token r, block b at half r*NB+b
        u32x4 v[VL];                    // V codes per read
        u32x4 vs[NB];                   // V scales: block b, tokens 0..7
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
    };

    // One 32-token tile starting at token tb, from its operands in registers.
    auto process = [&](const Ops &op, const int tb) {
        // ---------------- scores: S^T tile T, lane holds tokens 8j+4T+i, head n
        const uint32_t *ksc = op.ks;
        floatx4 sacc[2];
#pragma unroll
        for (int T = 0; T < 2; T++) {
            sacc[T] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int b = 0; b < NB; b++) {
                half8 ka;
                if (KT == KVQ_F16) {
                    const u32x4 w = op.k[T][b];
                    ka = pack4(w.x, w.y, w.z, w.w);
                } else if (KT == KVQ_Q8_0) {
                    ka = deq_q8(op.k[T][b].x, op.k[T][b].y);
                } else {
                    const uint32_t w = op.k[T][b].x;
                    ka = k_operand<KVQ_Q4_0>(&w);
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
        const bool tail = tb + TILE > t_end;
        uint32_t keep[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};  // per token pair
        if (tail) {
#pragma unroll
            for (int r = 0; r < 8; r++)
                if (tb + 8 * j + r >= t_end) {
                    x[r] = -INFINITY;
                    keep[r >> 1] &= (r & 1) ? 0x0000FFFFu : 0xFFFF0000u;
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
                // positions past the context may hold any bits: a masked pair
                // is forced to +0 instead of 0 * (scale bits)
                const u32x4 dv = op.vs[b];
                pb = pack4(h2_bits(bits_h2(p16[0]) * bits_h2(dv.x)) & keep[0],
                           h2_bits(bits_h2(p16[1]) * bits_h2(dv.y)) & keep[1],
                           h2_bits(bits_h2(p16[2]) * bits_h2(dv.z)) & keep[2],
                           h2_bits(bits_h2(p16[3]) * bits_h2(dv.w)) & keep[3]);
            }
            if (VT == KVQ_Q4_0) {
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
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    const int ct = 2 * b + hh;
                    half8 va;
                    const u32x4 w = op.v[ct];
                    if (VT == KVQ_F16) {
                        // a masked token's value may be any bits, even NaN
                        va = pack4(w.x & keep[0], w.y & keep[1], w.z & keep[2], w.w & keep[3]);
                    } else {
                        va = deq_q8(w.x, w.y);
                    }
                    o[ct] = mfma(va, pb, o[ct]);
                }
            }
        }
    };

    // ---------------- walk the split: this wave takes tiles wave, wave+4, ...
    // Per tile: wait for its copy, read its operands out of LDS into
    // registers, start copying the wave's next tile into the same LDS space,
    // then compute -- the copy of tile i+1 streams during the math of tile i.
    uint8_t *buf = lds_a + wave * g::BYTES;
    const int step = TILE * WAVES;
    int tb = t_begin + TILE * wave;
    if (tb < t_end) {
        issue_tile<KT, VT, D>(buf, tb, lane, doff, rs);
        while (true) {
            Ops op;
            read_ops(buf, op);
            const int tn = tb + step;
            if (tn < t_end) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS reads done before it is refilled
                issue_tile<KT, VT, D>(buf, tn, lane, doff, rs);
            }
            process(op, tb);
            tb = tn;
            if (tb >= t_end)
                break;
        }
    }
    // every copy into LDS has landed before the buffers are reused below
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---------------- merge the four waves: scale to the common max, then
    // accumulate in LDS one wave after the other (deterministic order)
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (j == 0)
        sm_m[wave][n] = m_run;
    __syncthreads();
    float M = sm_m[0][n];
#pragma unroll
    for (int w = 1; w < WAVES; w++)
        M = fmaxf(M, sm_m[w][n]);
    const float e = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
    if (j == 0)
        sm_l[wave][n] = l_tot * e;
    float *obuf = reinterpret_cast<float *>(lds_a);  // [16][D]
#pragma unroll
    for (int w = 0; w < WAVES; w++) {
        if (wave == w && n < G) {
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int idx = n * D + 16 * ct + 4 * j + i;
                    obuf[idx] = (w == 0 ? 0.0f : obuf[idx]) + o[ct][i] * e;
                }
        }
        __syncthreads();
    }

    const int Dp = D + 2;
    const int64_t head_stride = (int64_t)a.n_splits * Dp;  // between query heads
    float *ws_pair = a.ws + ((int64_t)s * a.Hq + (int64_t)h * G) * head_stride;
    float *out_pair = a.out + ((int64_t)s * a.Hq + (int64_t)h * G) * D;
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * WAVES) {
        const int gg = idx / D, c = idx - gg * D;
        float Mg = sm_m[0][gg], lsum = 0.0f;
#pragma unroll
        for (int w = 1; w < WAVES; w++)
            Mg = fmaxf(Mg, sm_m[w][gg]);
#pragma unroll
        for (int w = 0; w < WAVES; w++)
            lsum += sm_l[w][gg];
        const float acc = obuf[idx];
        if (nsp == 1) {
            out_pair[idx] = acc / lsum;  // the only split: final output
        } else {
            // device-scope stores: written through to the point where every
            // XCD's loads of the same scope see them, without flushing any L2
            float *dst = ws_pair + gg * head_stride + (int64_t)split * Dp;
            st_dev(dst + c, acc);
            if (c == 0) {
                st_dev(dst + D, Mg);
                st_dev(dst + D + 1, lsum);
            }
        }
    }
    if (nsp == 1)
        return;

    // ---------------- the last workgroup of this (sequence, kv head) merges
    // Every wave waits until its partial stores are performed (acknowledged at
    // device scope), then one lane counts the split as done; the workgroup
    // that completes the count merges.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.counters + pair, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = (prev == (unsigned)(nsp - 1));
    }
    __syncthreads();
    if (!sm_last)
        return;

    // (m_j, l_j) of every (split, head) into LDS (after the [16][D] buffer),
    // loads issued together; the host keeps nsp * G * 8 bytes within it
    float *wgt = reinterpret_cast<float *>(lds_a) + 16 * D;  // [nsp][G]: m_j, then 2^(m_j - M)
    float *lj = wgt + nsp * G;                               // [nsp][G]
    float *tot = &sm_m[0][0];                                // [16]: 1 / sum_j l_j 2^(m_j - M)
    for (int idx = threadIdx.x; idx < nsp * G; idx += 64 * WAVES) {
        const int sp = idx / G, gg = idx - sp * G;
        const float *pp = ws_pair + gg * head_stride + (int64_t)sp * Dp + D;
        wgt[idx] = ld_dev(pp);
        lj[idx] = ld_dev(pp + 1);
    }
    __syncthreads();
    if ((int)threadIdx.x < G) {
        const int gg = threadIdx.x;
        float Mx = -INFINITY;
        for (int sp = 0; sp < nsp; sp++)
            Mx = fmaxf(Mx, wgt[sp * G + gg]);
        float l = 0.0f;
        for (int sp = 0; sp < nsp; sp++) {
            const float ew = __builtin_amdgcn_exp2f(wgt[sp * G + gg] - Mx);
            wgt[sp * G + gg] = ew;
            l += lj[sp * G + gg] * ew;
        }
        tot[gg] = 1.0f / l;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * WAVES) {
        const int gg = idx / D, c = idx - gg * D;
        const float *base = ws_pair + gg * head_stride + c;
        float acc = 0.0f;
        int sp = 0;
        for (; sp + 8 <= nsp; sp += 8) {  // eight loads in flight at a time
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; u++)
                v[u] = ld_dev(base + (int64_t)(sp + u) * Dp);
#pragma unroll
            for (int u = 0; u < 8; u++)
                acc += v[u] * wgt[(sp + u) * G + gg];
        }
        for (; sp < nsp; sp++)
            acc += ld_dev(base + (int64_t)sp * Dp) * wgt[sp * G + gg];
        out_pair[idx] = acc * tot[gg];
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(a.counters + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int KT, int VT, int D>
hipError_t launch_dec(const DecodeArgs &a, int n_seqs, hipStream_t st)
{
    dim3 grid(a.n_splits, a.Hkv, n_seqs);
    hipLaunchKernelGGL((decode_kernel<KT, VT, D>), grid, dim3(64 * WAVES), 0, st, a);
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

template <int D>
int split_cap_d(int kt, int vt, int G)
{
    int bytes = 0;
#define KVQ_C(K, V) \
    if (kt == K && vt == V) bytes = Geo<K, V, D>::LDS_A;
    KVQ_C(KVQ_F16, KVQ_F16) KVQ_C(KVQ_F16, KVQ_Q8_0) KVQ_C(KVQ_F16, KVQ_Q4_0)
    KVQ_C(KVQ_Q8_0, KVQ_F16) KVQ_C(KVQ_Q8_0, KVQ_Q8_0) KVQ_C(KVQ_Q8_0, KVQ_Q4_0)
    KVQ_C(KVQ_Q4_0, KVQ_F16) KVQ_C(KVQ_Q4_0, KVQ_Q8_0) KVQ_C(KVQ_Q4_0, KVQ_Q4_0)
#undef KVQ_C
    // the merge keeps a [16][D] float buffer and (m_j, l_j) per (split, head)
    return (bytes - 16 * D * 4) / (8 * G);
}

}  // namespace

int decode_split_cap(int kt, int vt, int D, int G)
{
    int cap = D == 64 ? split_cap_d<64>(kt, vt, G) : D == 128 ? split_cap_d<128>(kt, vt, G) : split_cap_d<256>(kt, vt, G);
    return cap < KVQ_MAX_SPLITS ? cap : KVQ_MAX_SPLITS;
}

hipError_t launch_decode(int kt, int vt, int D, const DecodeArgs &a, int n_seqs, hipStream_t st)
{
    switch (D) {
    case 64: return launch_dec_d<64>(kt, vt, a, n_seqs, st);
    case 128: return launch_dec_d<128>(kt, vt, a, n_seqs, st);
    case 256: return launch_dec_d<256>(kt, vt, a, n_seqs, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
