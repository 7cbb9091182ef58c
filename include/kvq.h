/*
 * kvq.h -- C ABI of libkvq: a KV cache whose keys and values are stored at
 * independently chosen precisions (f16, q8_0, q5_0, q4_0; turbo3 for
 * values), with a quantizing
 * append and flash attention (decode and causal chunked prefill) that reads
 * the quantized blocks directly.  Built for AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *  - llama.cpp optimization guide "llama.cpp fuer Geschwindigkeit und
 *    Speicher optimieren" (docs.tokios.com), section "KV-Cache-Praezision":
 *    the cache types f16 / q8_0 / q4_0 and the fact that keys and values are
 *    set independently; section "Flash Attention": tiled attention that never
 *    materializes the score matrix and is exactly standard attention;
 *    section "Batch-Groessen-Abstimmung": prompts are processed in
 *    micro-batches (chunked prefill).
 *  - "KVSplit - 2- bis 3-mal laengerer Kontext auf Apple Silicon"
 *    (news.hada.io): sections "Zentrale Benchmark-Ergebnisse" and
 *    "Vergleich der Speicherersparnis" (K8V4 = 8-bit keys, 4-bit values;
 *    cache sizes at 8K tokens), "Roadmap" (separate quantization per layer).
 *  - llama.cpp issue "Eval bug: Metal fails mixed quantized KV on Apple
 *    Silicon when Flash Attention is unavailable ...": the llama_kv_cache
 *    size log lines (K q8_0 / V q4_0 byte totals) and, under "Expected
 *    behavior", the wish that an unusable configuration be refused up front,
 *    before anything has been set up -- this library's error convention
 *    (every argument is checked before any device work); and, in
 *    its comment thread, q5_0 named as the working middle ground between
 *    q8_0 and q4_0 (the format itself is not on the pages: ggml's 5-bit
 *    block, read the way q4_0 is read below).
 *  - "Benchmark TurboQuant en Apple Silicon" (asiai.dev), section "Que es
 *    TurboQuant?": values compressed to 3 bits after a random Walsh-Hadamard
 *    rotation and an optimal scalar quantizer, keys kept at q8_0 -- the
 *    values-only type turbo3 below (the format itself is a reading).
 *
 * Conventions for every entry point:
 *  - All tensors live in device memory owned by the caller; the library
 *    allocates nothing and is re-entrant (its only global state is a
 *    per-device cache of the compute-unit count, read once).
 *  - Per-sequence integer arrays (pos, ctx_len, q_pos0) are HOST arrays of
 *    n_seqs entries; they are validated on the host and passed to the
 *    kernels by value.
 *  - Every argument is validated on the host before anything is enqueued;
 *    on error a negative KVQ_E_* code is returned and no device work was
 *    issued.  KVQ_E_HIP reports a failed launch; faults inside a kernel
 *    surface at the caller's next synchronization.
 *  - `stream` is a hipStream_t (NULL = the default stream); all work is
 *    asynchronous on it and no host synchronization happens inside.
 *  - Device pointers must be 16-byte aligned.
 *  - Inputs must be finite: NaN/Inf inside K, V or Q is outside the
 *    contract and is not checked on the hot path.
 *
 * Storage layout of one layer's planes (the contract the CPU oracle
 * re-implements independently).  S = n_seqs, H = n_kv_heads,
 * D = head_dim, nb = D/32, Tc = max_ctx rounded up to a multiple of 32,
 * pair = s*H + h:
 *  - A 32-element block stores: f16: 32 binary16 values (64 B);
 *    q8_0: 32 int8 codes (32 B) + binary16 scale d, x^ = d*q;
 *    q4_0: 16 bytes, byte i = c_i | c_(i+16) << 4 (4-bit codes) + binary16
 *    scale d, x^ = d*(c-8); q5_0: 5-bit codes c, their low 4 bits packed as
 *    q4_0's, their fifth bits in a 32-bit word (bit i = element i), +
 *    binary16 scale d, x^ = d*(c-16); turbo3 (V planes only): 3-bit codes of
 *    the rotated block, their low 2 bits in 8 bytes (byte j: elements j,
 *    j+8, j+16, j+24 at bits 0, 2, 4, 6), their third bits in a 32-bit word
 *    (bit i = element i), + binary16 scale d (see Quantization).  Row code
 *    bytes R = 2D, D, D/2, D/2 (q5_0: the nibbles) or D/4 (turbo3: the
 *    2-bit planes); block b of a row occupies code bytes [b*R/nb, (b+1)*R/nb).
 *  - K plane ("token-major"): code byte r of token t at
 *        codes + (pair*Tc + t)*R + r;
 *    scale of block b at  scales + 2*((pair*Tc + t)*nb + b).
 *  - V plane ("8-token interleaved", so that one 8-byte or 16-byte load
 *    returns 8 consecutive tokens of one channel, the operand shape of the
 *    matrix-core P.V product): with unit size w = 2 bytes for f16 (one
 *    value) and 1 byte otherwise, U = R/w units per row, unit u of token t
 *    at  codes + w*((((pair*(Tc/8)) + t/8)*U + u)*8 + t%8);
 *    scale of block b at  scales + 2*(((pair*(Tc/8) + t/8)*nb + b)*8 + t%8).
 *  - q5_0 high-bit words and turbo3 third-bit words: in the codes allocation after the S*H*Tc*R bytes
 *    of rows, one little-endian uint32 per (token, block), at the index of
 *    that block's scale:  codes + S*H*Tc*R + 4*(scale index).
 *  - Plane bytes: codes S*H*Tc*R (+ S*H*Tc*nb*4 for q5_0 and turbo3), scales
 *    S*H*Tc*nb*2 (0 for f16).  With
 *    max_ctx a multiple of 32 nothing is padded: q8_0 costs 34 B and q4_0
 *    18 B per 32 elements, the sizes behind the KVSplit page's 176 / 93.5 /
 *    71.5 / 49.5 MiB and the issue's 816 + 432 MiB; q5_0 costs 22 B and
 *    turbo3 14 B (the TurboQuant page's ~4 GB KV at 32K tokens for a 70B
 *    model with q8_0 keys).
 *
 * Quantization (the ggml q8_0 / q4_0 block formats of the cache types named
 * on the llama.cpp pages), bit-exact, in binary32 unless stated:
 *  q8_0: amax = max|x|; d = f16(amax/127); id = d ? 1/d : 0;
 *        q = clamp(round_half_away(x*id), -127, 127).
 *  q4_0: m = the x of largest |x| (lowest index on ties, +0 if all zero);
 *        d = f16(m/-8); id = d ? 1/d : 0;
 *        c = clamp(trunc((x*id) + 8.5), 0, 15), product and sum rounded
 *        separately (no fused multiply-add).
 *  q5_0: as q4_0 with d = f16(m/-16) and c = clamp(trunc((x*id) + 16.5), 0, 31).
 *  turbo3: y = H*(s.x) for the 32x32 Sylvester Hadamard matrix H
 *        (H[k][i] = (-1)^popcount(k&i)) and s_i = -1 where bit i of
 *        0x9E3779B9 is set, exact (binary64 arithmetic); levels L = the
 *        8-level Lloyd-Max quantizer of N(0,1) in binary16 (+-0.2451,
 *        +-0.756, +-1.344, +-2.152); d = f16(f32(max|y|)/L[7]);
 *        id = d ? 1/d : 0; code = #{j : f32(y)*id >= (L[j]+L[j+1])/2};
 *        x^ = s.(H*(d*L[code]))/32.  Attention accumulates P.V in the
 *        rotated basis and rotates each output block back once.
 *  f16 (the conversion) rounds to nearest even.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache element types (llama.cpp's --cache-type-k / --cache-type-v values). */
typedef enum kvq_type { KVQ_F16 = 0, KVQ_Q8_0 = 1, KVQ_Q4_0 = 2, KVQ_Q5_0 = 3, KVQ_TURBO3 = 4 } kvq_type;

enum {
    KVQ_OK = 0,
    KVQ_E_ARG = -1,       /* NULL or misaligned pointer, malformed argument   */
    KVQ_E_TYPE = -2,      /* unknown type, type differs from the plane's, or
                             turbo3 on a K plane                              */
    KVQ_E_SHAPE = -3,     /* unsupported head_dim / head grouping / counts    */
    KVQ_E_RANGE = -4,     /* layer, position or context length out of range   */
    KVQ_E_WORKSPACE = -5, /* workspace NULL or smaller than required          */
    KVQ_E_HIP = -6,       /* a HIP call or kernel launch failed               */
    KVQ_E_TOO_BIG = -7    /* kvq_attn_decode_append_noalloc: the call needs
                             more partial slots than its static scratch holds */
};

/* Supported limits. */
#define KVQ_MAX_SEQS 256   /* n_seqs: per-sequence arrays travel as kernel args */
#define KVQ_MAX_GROUP 16   /* n_q_heads / n_kv_heads                            */
#define KVQ_MAX_SPLITS 256 /* decode context splits per (sequence, kv head)     */
/* head_dim must be 64, 128 or 256. */

typedef struct kvq_shape {
    int32_t n_layers;   /* >= 1                                  */
    int32_t n_seqs;     /* 1 .. KVQ_MAX_SEQS                     */
    int32_t n_q_heads;  /* multiple of n_kv_heads                */
    int32_t n_kv_heads; /* >= 1, n_q_heads/n_kv_heads <= 16      */
    int32_t head_dim;   /* 64, 128 or 256                        */
    int32_t max_ctx;    /* cache capacity in tokens, >= 1, with
                           max_ctx (rounded up to 32) * 2 * head_dim
                           < 2^31: one (sequence, kv head)'s range of
                           a stream is addressed with 32-bit offsets */
} kvq_shape;

/* One plane (the K or the V half of one layer). */
typedef struct kvq_plane {
    int32_t type;  /* kvq_type                                               */
    void *codes;   /* device, kvq_plane_bytes() codes bytes                  */
    void *scales;  /* device binary16 scales; NULL (and unused) for KVQ_F16  */
} kvq_plane;

/* The whole cache: k[l] and v[l] describe layer l (host arrays of
 * shape.n_layers planes; the types may differ per layer and per K/V). */
typedef struct kvq_cache {
    kvq_shape shape;
    const kvq_plane *k;
    const kvq_plane *v;
} kvq_cache;

/* Message for a KVQ_* code (static string, never NULL). */
const char *kvq_strerror(int code);

/* Bytes of one plane of `type` for `shape` (codes and scales separately).
 * Host only.  Errors: KVQ_E_ARG (NULL), KVQ_E_SHAPE, KVQ_E_TYPE. */
int kvq_plane_bytes(const kvq_shape *shape, int32_t type, size_t *codes_bytes, size_t *scale_bytes);

/* Validate a cache descriptor on the host (shape limits, types, non-NULL and
 * aligned plane pointers).  No device access. */
int kvq_cache_check(const kvq_cache *cache);

/* Quantize n_new new rows per sequence into layer `layer` at positions
 * pos[s] .. pos[s]+n_new-1 (the quantizing row copy into the cache that the
 * llama.cpp issue names "CPY").
 *   K, V : device binary16 [n_seqs][n_new][n_kv_heads][head_dim]
 *   pos  : host int32 [n_seqs], 0 <= pos[s], pos[s] + n_new <= max_ctx
 *   k_type, v_type must equal the layer's plane types (else KVQ_E_TYPE).
 * Rows outside the written range are untouched.  One kernel launch. */
int kvq_append(const kvq_cache *cache, int32_t layer, const void *K, const void *V, int32_t n_new,
               const int32_t *pos, int32_t k_type, int32_t v_type, void *stream);

/* Workspace bytes that kvq_attn_decode (and kvq_attn_decode_append) need for
 * any ctx_len <= max_ctx and any n_splits: one 32-bit counter per (sequence,
 * kv head) pair (padded to 256 bytes), then one partial slot of
 * (n_q_heads/n_kv_heads) * (head_dim+4) floats per workgroup of four waves,
 * for the most workgroups a call can use (see kvq_attn_decode).
 * The workspace must be zero-filled before its first use (the counters start
 * at zero); every call leaves them zero again, so it is cleared once, not per
 * call.  A workspace belongs to caches of one shape, and serves one call at a
 * time: calls that overlap in time (other streams) need workspaces of their
 * own. */
int kvq_decode_workspace_bytes(const kvq_shape *shape, size_t *bytes);

/* Flash-decode one query token per sequence over layer `layer`: tiled,
 * exact softmax attention that never materializes the score row (the
 * llama.cpp guide, section "Flash Attention"), read straight from the
 * quantized blocks.  With one query token per sequence there is little
 * parallel work per (sequence, kv head), so the context of each pair is
 * split over several waves whose partial results are combined by a
 * log-sum-exp merge; that split is this library's design (the pages do not
 * describe one).
 *   Q       : device binary16 [n_seqs][n_q_heads][head_dim]
 *   ctx_len : host int32 [n_seqs], 1 <= ctx_len[s] <= max_ctx; query s
 *             attends to cache positions 0 .. ctx_len[s]-1 (append the new
 *             token's K/V first: ctx_len counts it)
 *   scale   : multiplies Q.K (typically 1/sqrt(head_dim)), used as passed
 *   out     : device float32 [n_seqs][n_q_heads][head_dim]
 *   workspace, workspace_bytes: device scratch for the partials and the
 *             merge counters (zero-filled before the first call, see
 *             kvq_decode_workspace_bytes)
 *   n_splits: how many waves share the context of one (sequence, kv head)
 *             pair; 0 chooses: four waves per compute unit over the whole
 *             batch (eight where K is q5_0, V is q5_0 or turbo3, or both are
 *             q4_0 -- neither half f16 -- at head_dim <= 128 while each wave
 *             still gets at least 16 tiles); each pair of a sequence with nt
 *             tiles gets ceil(nt / tau) waves, rounded up to a multiple of
 *             four, for the smallest tau >= 4 that keeps the total within
 *             that, so that no wave streams more than tau tiles whatever the
 *             mix of contexts.  Never more than the pair's 32-token tiles,
 *             nor more than KVQ_MAX_SPLITS.
 * Query head hq reads kv head hq / (n_q_heads/n_kv_heads).  One launch on
 * `stream`.  The k waves of a pair, in workgroups of four, take its tiles
 * round robin (wave r: tiles r, r+k, ...); the four waves of a workgroup
 * combine their (max, sum, unnormalized output) partials, and the pair's
 * last workgroup to finish combines the workgroups' partials (log-sum-exp,
 * in a fixed order: results are bitwise repeatable) into `out`.  Errors:
 * KVQ_E_RANGE (ctx_len, n_splits > KVQ_MAX_SPLITS), KVQ_E_WORKSPACE,
 * KVQ_E_SHAPE (2^23 or more workgroups). */
int kvq_attn_decode(const kvq_cache *cache, int32_t layer, const void *Q, const int32_t *ctx_len, float scale,
                    float *out, void *workspace, size_t workspace_bytes, int32_t n_splits, void *stream);

/* One decode step of layer `layer` with the new token's append folded in:
 * quantizes K[s], V[s] into position ctx_len[s]-1 and then attends as
 * kvq_attn_decode does.  The planes and `out` come out bit-identical to
 * kvq_append(n_new = 1, pos[s] = ctx_len[s]-1) followed by kvq_attn_decode
 * with the same arguments (same quantizer, same work split), with one launch
 * fewer: the wave that reads a pair's last tile writes the row before it
 * copies that tile.
 *   K, V : device binary16 [n_seqs][n_kv_heads][head_dim], 16-byte aligned
 * Other arguments and errors as kvq_attn_decode.  The rows of K and V must
 * not overlap the cache planes. */
int kvq_attn_decode_append(const kvq_cache *cache, int32_t layer, const void *K, const void *V, const void *Q,
                           const int32_t *ctx_len, float scale, float *out, void *workspace,
                           size_t workspace_bytes, int32_t n_splits, void *stream);

/* Causal attention for a chunk of n_tok queries per sequence whose K/V rows
 * are already appended at positions q_pos0[s] .. q_pos0[s]+n_tok-1 (the
 * micro-batch of the llama.cpp guide's "Batch-Groessen-Abstimmung").
 *   Q      : device binary16 [n_seqs][n_tok][n_q_heads][head_dim]
 *   q_pos0 : host int32 [n_seqs], 0 <= q_pos0[s], q_pos0[s]+n_tok <= max_ctx
 *   out    : device float32 [n_seqs][n_tok][n_q_heads][head_dim]
 * Query i of sequence s attends to positions 0 .. q_pos0[s]+i; cache bytes
 * past q_pos0[s]+n_tok-1 may hold anything.  One launch on `stream`.
 * Errors: the cache checks of kvq_cache_check, KVQ_E_RANGE (layer, n_tok < 1
 * or a chunk past max_ctx), KVQ_E_ARG (NULL or misaligned Q / out / q_pos0,
 * non-finite scale). */
int kvq_attn_prefill_chunk(const kvq_cache *cache, int32_t layer, const void *Q, int32_t n_tok,
                           const int32_t *q_pos0, float scale, float *out, void *stream);

/* ---- for callers that cannot allocate device memory ----
 *
 * kvq_attn_decode_append without the workspace argument, for callers that
 * cannot call hipMalloc or allocate through a library: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The
 * partial slots live in a static device array of KVQ_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends; its
 * device address is looked up once per device, at the first call on that
 * device (with that device current).  Nothing is allocated by any call.
 *   - The array holds the merge counters of up to KVQ_NOALLOC_MAX_PAIRS
 *     (sequence, kv head) pairs (32 KiB), then the partial slots: one of
 *     (n_q_heads/n_kv_heads) x (head_dim+4) floats per workgroup of the
 *     call's work split.  A call with more pairs, or more slots than the
 *     rest of the array holds, returns KVQ_E_TOO_BIG before any device work.
 *     At group 8 and head_dim 128 (4224 B a slot) that is 3964 workgroups:
 *     more than the automatic split of a 256-CU device uses for any batch.
 *   - The first call on a device also enqueues a small kernel that zeroes
 *     the counter region; every call leaves the counters zero.  Every call
 *     on one GPU shares that GPU's array, which keeps the last call's
 *     partials.  Calls that overlap in time on one GPU (other streams, other
 *     threads) race on the array and must not be issued; calls ordered on one
 *     stream are safe.
 * Other arguments, results and errors as kvq_attn_decode_append; for the
 * same arguments and n_splits the planes and `out` are bit-identical. */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
#define KVQ_NOALLOC_MAX_PAIRS 8192 /* n_seqs * n_kv_heads of a call */
int kvq_attn_decode_append_noalloc(const kvq_cache *cache, int32_t layer, const void *K, const void *V,
                                   const void *Q, const int32_t *ctx_len, float scale, float *out,
                                   int32_t n_splits, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
