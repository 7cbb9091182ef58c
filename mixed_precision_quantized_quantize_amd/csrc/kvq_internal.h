// kvq_internal.h -- kernel argument blocks and launchers shared by the host
// validation layer (kvq_api.cpp) and the HIP kernels (*.hip).  Not part of
// the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// Plane capacity in tokens: a whole number of 32-token tiles, so that a
// kernel reading a full tile never leaves the plane.
__host__ __device__ inline int64_t capacity(int64_t max_ctx) { return (max_ctx + 31) / 32 * 32; }

__host__ __device__ constexpr int64_t row_code_bytes(int type, int64_t D)
{
    // q4_0 and the q5_0 nibbles: D/2; turbo3's 2-bit planes: D/4
    return type == KVQ_F16 ? 2 * D : type == KVQ_Q8_0 ? D : type == KVQ_TURBO3 ? D / 4 : D / 2;
}

// Types whose code allocation continues with one 32-bit word per (row, block).
__host__ __device__ constexpr bool has_bit_words(int type) { return type == KVQ_Q5_0 || type == KVQ_TURBO3; }

// Every (K type, V type) pair, for the kernels' dispatch tables.
// (turbo3 is a values-only type.)
#define KVQ_FOR_EACH_TYPE_PAIR(X)                                                                  \
    X(KVQ_F16, KVQ_F16) X(KVQ_F16, KVQ_Q8_0) X(KVQ_F16, KVQ_Q4_0) X(KVQ_F16, KVQ_Q5_0)             \
    X(KVQ_Q8_0, KVQ_F16) X(KVQ_Q8_0, KVQ_Q8_0) X(KVQ_Q8_0, KVQ_Q4_0) X(KVQ_Q8_0, KVQ_Q5_0)         \
    X(KVQ_Q4_0, KVQ_F16) X(KVQ_Q4_0, KVQ_Q8_0) X(KVQ_Q4_0, KVQ_Q4_0) X(KVQ_Q4_0, KVQ_Q5_0)         \
    X(KVQ_Q5_0, KVQ_F16) X(KVQ_Q5_0, KVQ_Q8_0) X(KVQ_Q5_0, KVQ_Q4_0) X(KVQ_Q5_0, KVQ_Q5_0)         \
    X(KVQ_F16, KVQ_TURBO3) X(KVQ_Q8_0, KVQ_TURBO3) X(KVQ_Q4_0, KVQ_TURBO3) X(KVQ_Q5_0, KVQ_TURBO3)

struct AppendArgs {
    const uint16_t *src[2];  // K, V binary16 [S][n_new][H][D]
    uint8_t *codes[2];       // K plane, V plane
    uint16_t *scales[2];
    uint32_t *qh[2];         // q5_0 high-bit / turbo3 third-bit words (after the rows), else NULL
    int32_t H, D, Tc, n_new, n_seqs;
    int32_t ng;  // 8-token groups per sequence the V plane's launch covers (the most any sequence spans)
    int32_t pos[KVQ_MAX_SEQS];
};

// Decode work split: every (sequence, kv head) pair of sequence s gets k[s]
// waves in kw_s = ceil(k[s]/4) workgroups of four; wave r = 4*rw + w (of
// workgroup rw) streams the pair's tiles r, r + k, ...  The pairs are
// interleaved over the grid: with one kw for all sequences (kw_uniform)
// workgroup rw of pair p is workgroup rw*pairs + p; otherwise workgroup
// wg_start[s] + rw*n_kv_heads + h.  wg_start[s] = first workgroup of
// sequence s (n_kv_heads * the kw of every earlier sequence); wg_start[n_seqs]
// = n_wg.  A pair's workgroups merge through one slot each in `ws` (at the
// workgroup's index) and the pair's counter in `counters`.
constexpr int KVQ_MAX_WG_PER_PAIR = KVQ_MAX_SPLITS / 4;  // k <= KVQ_MAX_SPLITS waves per pair

struct DecodeArgs {
    const uint8_t *kc;
    const uint16_t *ks;
    const uint8_t *vc;
    const uint16_t *vs;
    const uint16_t *q;    // [S][Hq][D]
    const uint32_t *kqh, *vqh;    // q5_0 high-bit / turbo3 third-bit words, else NULL
    const uint16_t *knew, *vnew;  // NULL, or the new row of every sequence, binary16 [S][Hkv][D],
                                  // to quantize into position ctx_len[s] - 1 first
    float *out;           // [S][Hq][D]
    float *ws;            // slots [n_wg][G][D+4]: O (unnormalized), m (base 2), l
    uint32_t *counters;   // one per (sequence, kv head) pair, zero between calls
    int32_t Hq, Hkv, G, Tc, n_seqs, n_wg;
    int32_t kw_uniform;  // workgroups per pair when every sequence has the same count, else 0
    float c2;  // scale * log2(e)
    int32_t ctx_len[KVQ_MAX_SEQS];
    int32_t wg_start[KVQ_MAX_SEQS + 1];
    int16_t k[KVQ_MAX_SEQS];  // waves per pair of each sequence
};

struct PrefillArgs {
    const uint8_t *kc;
    const uint16_t *ks;
    const uint8_t *vc;
    const uint16_t *vs;
    const uint32_t *kqh, *vqh;  // q5_0 high-bit words, else NULL
    const uint16_t *q;  // [S][n_tok][Hq][D]
    float *out;         // [S][n_tok][Hq][D]
    int32_t Hq, Hkv, G, Tc, n_tok, n_seqs;
    int32_t gp_log2;  // rows of one query token: the group padded to 2^gp_log2
    float c2;
    int32_t q_pos0[KVQ_MAX_SEQS];
};

// Launchers return hipSuccess or the launch error.
hipError_t launch_append(int k_type, int v_type, const AppendArgs &a, int n_quads, hipStream_t st);
// One launch: streaming, then the in-kernel merge.
hipError_t launch_decode(int k_type, int v_type, int D, const DecodeArgs &a, hipStream_t st);
hipError_t launch_prefill(int k_type, int v_type, int D, const PrefillArgs &a, hipStream_t st);

}  // namespace kvq
