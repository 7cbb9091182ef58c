// kvq_api.cpp -- the C ABI of libkvq: host-side validation and dispatch.
//
// Every argument is checked here before anything is enqueued, so a failing
// call returns a KVQ_E_* code with no device side effects: an unusable
// configuration is refused up front, before anything is set up, as the
// llama.cpp issue "Eval bug: Metal fails mixed quantized KV on Apple Silicon
// when Flash Attention is unavailable" wishes under "Expected behavior".  The
// kernels themselves assume the checked preconditions.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kvq_internal.h"

using namespace kvq;

// Partial slots of kvq_attn_decode_append_noalloc: a static array that every
// GPU the library runs on holds until the process ends.  In host code this
// name is only a host-side stand-in; the array's device address on the
// current device comes from noalloc_scratch() below and is what the kernels
// receive.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;

// The scratch array starts with a fixed region of counters for up to
// KVQ_NOALLOC_MAX_PAIRS (sequence, kv head) pairs, whatever the shape of a
// call, so that one call's slots never land where another call's counters
// are; the slots follow it.
constexpr size_t NOALLOC_COUNTER_BYTES = (size_t)KVQ_NOALLOC_MAX_PAIRS * 4;

__global__ void zero_words(uint32_t *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

// The array's address on the current device, looked up once per device (with
// that device current) and kept: each GPU holds its own copy of the array at
// its own address.  The first call on a device also clears the counter
// region (a small kernel on the caller's stream; every later call leaves the
// counters zero).  KVQ_E_HIP if the lookup or the launch fails.
int noalloc_scratch(void **ptr, void *stream)
{
    static std::mutex mu;
    static void *addr[MAX_DEVICES] = {nullptr};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return KVQ_E_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return KVQ_E_HIP;
        hipLaunchKernelGGL(zero_words, dim3((KVQ_NOALLOC_MAX_PAIRS + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                           (uint32_t *)p, KVQ_NOALLOC_MAX_PAIRS);
        if (hipGetLastError() != hipSuccess)
            return KVQ_E_HIP;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return KVQ_OK;
}

bool valid_type(int32_t t)
{
    return t == KVQ_F16 || t == KVQ_Q8_0 || t == KVQ_Q4_0 || t == KVQ_Q5_0 || t == KVQ_TURBO3;
}

// q5_0's high-bit words follow the nibble rows in the codes allocation.
uint32_t *high_bits(const kvq_shape &sh, const kvq_plane &p)
{
    if (!has_bit_words(p.type))
        return nullptr;
    const int64_t rows = (int64_t)sh.n_seqs * sh.n_kv_heads * capacity(sh.max_ctx);
    return reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(p.codes) + rows * row_code_bytes(p.type, sh.head_dim));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const kvq_shape *sh)
{
    if (!sh)
        return KVQ_E_ARG;
    if (sh->n_layers < 1 || sh->n_seqs < 1 || sh->n_seqs > KVQ_MAX_SEQS || sh->n_kv_heads < 1 ||
        sh->n_q_heads < 1 || sh->max_ctx < 1)
        return KVQ_E_SHAPE;
    if (sh->head_dim != 64 && sh->head_dim != 128 && sh->head_dim != 256)
        return KVQ_E_SHAPE;
    if (sh->n_q_heads % sh->n_kv_heads != 0 || sh->n_q_heads / sh->n_kv_heads > KVQ_MAX_GROUP)
        return KVQ_E_SHAPE;
    // byte offsets inside one plane must fit comfortably in 63 bits, and the
    // grid dimensions in their hardware limits
    if ((int64_t)sh->n_seqs * sh->n_kv_heads * capacity(sh->max_ctx) > ((int64_t)1 << 40))
        return KVQ_E_SHAPE;
    // the kernels address one (sequence, kv head)'s range of a stream with
    // 32-bit offsets: its largest stream (binary16 rows, 2*head_dim bytes a
    // token) must stay below 2^31 bytes
    if (capacity(sh->max_ctx) * 2 * sh->head_dim >= ((int64_t)1 << 31))
        return KVQ_E_SHAPE;
    return KVQ_OK;
}

int check_plane(const kvq_plane *p)
{
    if (!valid_type(p->type))
        return KVQ_E_TYPE;
    if (!p->codes || !aligned16(p->codes))
        return KVQ_E_ARG;
    if (p->type != KVQ_F16 && (!p->scales || !aligned16(p->scales)))
        return KVQ_E_ARG;
    return KVQ_OK;
}

int check_cache(const kvq_cache *c)
{
    if (!c)
        return KVQ_E_ARG;
    int rc = check_shape(&c->shape);
    if (rc)
        return rc;
    if (!c->k || !c->v)
        return KVQ_E_ARG;
    for (int l = 0; l < c->shape.n_layers; l++) {
        if ((rc = check_plane(&c->k[l])) || (rc = check_plane(&c->v[l])))
            return rc;
        if (c->k[l].type == KVQ_TURBO3)  // a values-only type
            return KVQ_E_TYPE;
    }
    return KVQ_OK;
}

int check_layer(const kvq_cache *c, int32_t layer)
{
    int rc = check_cache(c);
    if (rc)
        return rc;
    if (layer < 0 || layer >= c->shape.n_layers)
        return KVQ_E_RANGE;
    return KVQ_OK;
}

// Decode work split (the kernels describe it): k waves per (sequence, kv
// head) pair, the same k for the pairs of one sequence.  n_splits > 0 asks
// for k = n_splits; 0 fills the device (waves_per_cu waves per CU, every
// wave at most tau tiles for the smallest tau >= 4 that fits, see
// decode_plan).  Never more waves for a pair than it has tiles.
constexpr int AUTO_WAVES_MAX = 4096;
// Waves per CU of the automatic split.  Where the tile math is heavy for its
// bytes (K q4_0 or q5_0, or V q5_0 or turbo3: more vector instructions to
// unpack the codes) two workgroups of four waves share a CU, so that one
// wave's math overlaps another's copies: measured about 25% faster for
// q4_0/q4_0, q5_0/q5_0 and q8_0/turbo3 at head_dim 128 -- as long as each
// wave still gets at least 16 tiles (a one-sequence 70B-shaped layer with
// turbo3 values, 4 tiles per wave at eight waves per CU: 30 us against 26.5
// with four).  Otherwise one workgroup per CU, which streams best (K8V4: 6%
// faster than two).  One at head_dim 256 either way: its waves need all 512
// registers.  `tiles`: the call's (kv head, tile) units.
int waves_per_cu(const kvq_shape &sh, int32_t kt, int32_t vt, int64_t tiles, int cus)
{
    if (sh.head_dim > 128)
        return 4;
    // Measured over all 20 pairs at the Llama-3-8B shape: q4_0 keys are heavy
    // only beside 4- or 5-bit or turbo3 values (q4_0/q8_0: 138 us with four,
    // 150 with eight), and a binary16 half makes any pair byte-heavy again
    // (f16/q5_0, q5_0/f16, f16/turbo3: 3-6% faster with four).
    const bool heavy = (kt == KVQ_Q5_0 || vt == KVQ_Q5_0 || vt == KVQ_TURBO3 || (kt == KVQ_Q4_0 && vt == KVQ_Q4_0)) &&
                       kt != KVQ_F16 && vt != KVQ_F16;
    return heavy && tiles >= (int64_t)16 * 8 * cus ? 8 : 4;
}

int device_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

// Plans a decode call: k[s] waves per pair of sequence s, in kw_s =
// ceil(k[s]/4) workgroups; fills wg_start[0..n_seqs] and *kw_uniform (the
// workgroups per pair when all sequences have the same count, else 0) and
// returns the workgroup count.  Never more waves for a pair than it has
// tiles, nor more than KVQ_MAX_SPLITS.
int64_t decode_plan(const kvq_shape &sh, int32_t kt, int32_t vt, const int32_t *ctx_len, int32_t req,
                    int32_t *wg_start, int16_t *k_out, int32_t *kw_uniform)
{
    int64_t T = 0;
    for (int s = 0; s < sh.n_seqs; s++)
        T += (int64_t)sh.n_kv_heads * ((ctx_len[s] + 31) / 32);
    const int cus = device_cus();
    const int64_t target = std::min<int64_t>((int64_t)cus * waves_per_cu(sh, kt, vt, T, cus), AUTO_WAVES_MAX);
    // Automatic split: the fewest tiles per wave, tau >= 4, for which
    // k_s = ceil(nt_s / tau) waves per pair stay within the target -- every
    // wave then streams at most tau tiles, whatever the mix of contexts (a
    // share proportional to the context, rounded down, left a short
    // sequence's single wave with up to twice the average).
    int64_t tau = 0;
    if (req <= 0) {
        int64_t nt_max = 1;
        for (int s = 0; s < sh.n_seqs; s++)
            nt_max = std::max<int64_t>(nt_max, (ctx_len[s] + 31) / 32);
        auto waves = [&](int64_t t) {
            int64_t w = 0;
            for (int s = 0; s < sh.n_seqs; s++)
                w += ((ctx_len[s] + 31) / 32 + t - 1) / t * sh.n_kv_heads;
            return w;
        };
        int64_t lo = std::max<int64_t>(4, (T + target - 1) / target), hi = std::max(lo, nt_max);
        while (lo < hi) {  // smallest tau in [lo, hi] whose waves fit (hi when none does)
            const int64_t mid = (lo + hi) / 2;
            if (waves(mid) <= target)
                hi = mid;
            else
                lo = mid + 1;
        }
        tau = lo;
    }
    int64_t n_wg = 0;
    for (int s = 0; s < sh.n_seqs; s++) {
        const int64_t nt = (ctx_len[s] + 31) / 32;
        int64_t k = req > 0 ? req : (nt + tau - 1) / tau;
        if (req <= 0)
            k = (k + 3) / 4 * 4;  // whole workgroups of four waves where the tiles allow
        k = std::max<int64_t>(1, std::min<int64_t>({k, nt, (int64_t)KVQ_MAX_SPLITS}));
        const int64_t kw = (k + 3) / 4;
        k_out[s] = (int16_t)k;
        if (s == 0)
            *kw_uniform = (int32_t)kw;
        else if (*kw_uniform != kw)
            *kw_uniform = 0;
        wg_start[s] = (int32_t)n_wg;
        n_wg += kw * sh.n_kv_heads;
    }
    wg_start[sh.n_seqs] = (int32_t)n_wg;
    return n_wg;
}

// Workspace: one counter per (sequence, kv head) pair (zero between calls),
// padded to 256 bytes, then one slot of [G][head_dim + 4] floats per
// workgroup.
size_t counters_bytes(const kvq_shape &sh) { return ((size_t)sh.n_seqs * sh.n_kv_heads * 4 + 255) / 256 * 256; }

size_t slot_bytes(const kvq_shape &sh, int64_t n_wg)
{
    const int64_t G = sh.n_q_heads / sh.n_kv_heads;
    return (size_t)(n_wg * G * (sh.head_dim + 4) * (int64_t)sizeof(float));
}

size_t workspace_need(const kvq_shape &sh, int64_t n_wg) { return counters_bytes(sh) + slot_bytes(sh, n_wg); }

}  // namespace

extern "C" {

const char *kvq_strerror(int code)
{
    switch (code) {
    case KVQ_OK: return "ok";
    case KVQ_E_ARG: return "invalid argument (NULL or misaligned pointer, malformed value)";
    case KVQ_E_TYPE: return "unknown cache type, or type does not match the layer's plane";
    case KVQ_E_SHAPE: return "unsupported shape (head_dim 64/128/256, n_q_heads multiple of n_kv_heads, group <= 16, n_seqs <= 256)";
    case KVQ_E_RANGE: return "layer, position or context length out of range";
    case KVQ_E_WORKSPACE: return "workspace missing or too small";
    case KVQ_E_HIP: return "HIP launch failed";
    case KVQ_E_TOO_BIG: return "the call needs more partial slots than the no-allocation entry point's static scratch holds (KVQ_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown kvq error code";
    }
}

int kvq_plane_bytes(const kvq_shape *shape, int32_t type, size_t *codes_bytes, size_t *scale_bytes)
{
    int rc = check_shape(shape);
    if (rc)
        return rc;
    if (!codes_bytes || !scale_bytes)
        return KVQ_E_ARG;
    if (!valid_type(type))
        return KVQ_E_TYPE;
    const int64_t rows = (int64_t)shape->n_seqs * shape->n_kv_heads * capacity(shape->max_ctx);
    *codes_bytes = (size_t)(rows * row_code_bytes(type, shape->head_dim));
    if (has_bit_words(type))
        *codes_bytes += (size_t)(rows * (shape->head_dim / 32) * 4);
    *scale_bytes = (type == KVQ_F16) ? 0 : (size_t)(rows * (shape->head_dim / 32) * 2);
    return KVQ_OK;
}

int kvq_cache_check(const kvq_cache *cache) { return check_cache(cache); }

int kvq_append(const kvq_cache *cache, int32_t layer, const void *K, const void *V, int32_t n_new,
               const int32_t *pos, int32_t k_type, int32_t v_type, void *stream)
{
    int rc = check_layer(cache, layer);
    if (rc)
        return rc;
    const kvq_shape &sh = cache->shape;
    if (!K || !V || !pos || !aligned16(K) || !aligned16(V))
        return KVQ_E_ARG;
    if (!valid_type(k_type) || !valid_type(v_type))
        return KVQ_E_TYPE;
    if (k_type != cache->k[layer].type || v_type != cache->v[layer].type)
        return KVQ_E_TYPE;
    if (n_new < 1)
        return KVQ_E_RANGE;
    for (int s = 0; s < sh.n_seqs; s++)
        if (pos[s] < 0 || (int64_t)pos[s] + n_new > sh.max_ctx)
            return KVQ_E_RANGE;
    const int64_t n_quads = (int64_t)sh.n_seqs * n_new * sh.n_kv_heads * (sh.head_dim / 32);
    if (n_quads > ((int64_t)1 << 31) - 64)
        return KVQ_E_SHAPE;

    AppendArgs a;
    memset(&a, 0, sizeof(a));
    a.src[0] = (const uint16_t *)K;
    a.src[1] = (const uint16_t *)V;
    a.codes[0] = (uint8_t *)cache->k[layer].codes;
    a.codes[1] = (uint8_t *)cache->v[layer].codes;
    a.scales[0] = (uint16_t *)cache->k[layer].scales;
    a.scales[1] = (uint16_t *)cache->v[layer].scales;
    a.qh[0] = high_bits(sh, cache->k[layer]);
    a.qh[1] = high_bits(sh, cache->v[layer]);
    a.H = sh.n_kv_heads;
    a.D = sh.head_dim;
    a.Tc = (int32_t)capacity(sh.max_ctx);
    a.n_new = n_new;
    a.n_seqs = sh.n_seqs;
    memcpy(a.pos, pos, sizeof(int32_t) * sh.n_seqs);
    // the V plane is written in 8-token groups: the most groups any
    // sequence's range [pos, pos + n_new) touches
    int64_t ng = 1;
    for (int s = 0; s < sh.n_seqs; s++)
        ng = std::max<int64_t>(ng, (pos[s] % 8 + (int64_t)n_new + 7) / 8);
    if ((int64_t)sh.n_seqs * sh.n_kv_heads * ng > ((int64_t)1 << 31) - 64)
        return KVQ_E_SHAPE;
    a.ng = (int32_t)ng;
    hipError_t e = launch_append(k_type, v_type, a, (int)n_quads, (hipStream_t)stream);
    return e == hipSuccess ? KVQ_OK : KVQ_E_HIP;
}

int kvq_decode_workspace_bytes(const kvq_shape *shape, size_t *bytes)
{
    int rc = check_shape(shape);
    if (rc)
        return rc;
    if (!bytes)
        return KVQ_E_ARG;
    // the most workgroups any call can use: per pair ceil(k/4) for at most
    // min(tiles of a full cache, KVQ_MAX_SPLITS) waves
    const int64_t pairs = (int64_t)shape->n_seqs * shape->n_kv_heads;
    const int64_t nt_max = capacity(shape->max_ctx) / 32;
    const int64_t kw_max = (std::min<int64_t>(nt_max, KVQ_MAX_SPLITS) + 3) / 4;
    *bytes = workspace_need(*shape, pairs * kw_max);
    return KVQ_OK;
}

}  // extern "C"

namespace {

// noalloc: the partial slots go into the static scratch array instead of
// `workspace` (which is then ignored).
int attn_decode(const kvq_cache *cache, int32_t layer, const void *K, const void *V, const void *Q,
                const int32_t *ctx_len, float scale, float *out, void *workspace, size_t workspace_bytes,
                int32_t n_splits, void *stream, bool noalloc = false)
{
    int rc = check_layer(cache, layer);
    if (rc)
        return rc;
    const kvq_shape &sh = cache->shape;
    if (!Q || !ctx_len || !out || !aligned16(Q) || !aligned16(out))
        return KVQ_E_ARG;
    if (!isfinite(scale))
        return KVQ_E_ARG;
    if (n_splits < 0 || n_splits > KVQ_MAX_SPLITS)
        return KVQ_E_RANGE;
    DecodeArgs a;
    memset(&a, 0, sizeof(a));
    for (int s = 0; s < sh.n_seqs; s++)
        if (ctx_len[s] < 1 || ctx_len[s] > sh.max_ctx)
            return KVQ_E_RANGE;
    const int64_t n_wg = decode_plan(sh, cache->k[layer].type, cache->v[layer].type, ctx_len, n_splits, a.wg_start,
                                     a.k, &a.kw_uniform);
    if (n_wg >= ((int64_t)1 << 31) / 256)
        return KVQ_E_SHAPE;
    size_t counter_region = counters_bytes(sh);
    if (noalloc) {
        if ((int64_t)sh.n_seqs * sh.n_kv_heads > KVQ_NOALLOC_MAX_PAIRS ||
            NOALLOC_COUNTER_BYTES + slot_bytes(sh, n_wg) > KVQ_NOALLOC_SCRATCH_BYTES)
            return KVQ_E_TOO_BIG;
        if ((rc = noalloc_scratch(&workspace, stream)) != KVQ_OK)
            return rc;
        workspace_bytes = KVQ_NOALLOC_SCRATCH_BYTES;
        counter_region = NOALLOC_COUNTER_BYTES;
    }
    if (!workspace || !aligned16(workspace) || workspace_bytes < counter_region + slot_bytes(sh, n_wg))
        return KVQ_E_WORKSPACE;

    const kvq_plane &kp = cache->k[layer], &vp = cache->v[layer];
    a.kc = (const uint8_t *)kp.codes;
    a.ks = (const uint16_t *)kp.scales;
    a.vc = (const uint8_t *)vp.codes;
    a.vs = (const uint16_t *)vp.scales;
    a.kqh = high_bits(sh, kp);
    a.vqh = high_bits(sh, vp);
    a.q = (const uint16_t *)Q;
    a.knew = (const uint16_t *)K;
    a.vnew = (const uint16_t *)V;
    a.out = out;
    a.counters = (uint32_t *)workspace;
    a.ws = (float *)((uint8_t *)workspace + counter_region);
    a.Hq = sh.n_q_heads;
    a.Hkv = sh.n_kv_heads;
    a.G = sh.n_q_heads / sh.n_kv_heads;
    a.Tc = (int32_t)capacity(sh.max_ctx);
    a.n_seqs = sh.n_seqs;
    a.n_wg = (int32_t)n_wg;
    a.c2 = (float)((double)scale * 1.4426950408889634);
    memcpy(a.ctx_len, ctx_len, sizeof(int32_t) * sh.n_seqs);
    hipError_t e = launch_decode(kp.type, vp.type, sh.head_dim, a, (hipStream_t)stream);
    return e == hipSuccess ? KVQ_OK : KVQ_E_HIP;
}

}  // namespace

extern "C" {

int kvq_attn_decode(const kvq_cache *cache, int32_t layer, const void *Q, const int32_t *ctx_len, float scale,
                    float *out, void *workspace, size_t workspace_bytes, int32_t n_splits, void *stream)
{
    return attn_decode(cache, layer, nullptr, nullptr, Q, ctx_len, scale, out, workspace, workspace_bytes, n_splits,
                       stream);
}

int kvq_attn_decode_append(const kvq_cache *cache, int32_t layer, const void *K, const void *V, const void *Q,
                           const int32_t *ctx_len, float scale, float *out, void *workspace,
                           size_t workspace_bytes, int32_t n_splits, void *stream)
{
    if (!K || !V || !aligned16(K) || !aligned16(V))
        return KVQ_E_ARG;
    return attn_decode(cache, layer, K, V, Q, ctx_len, scale, out, workspace, workspace_bytes, n_splits, stream);
}

int kvq_attn_decode_append_noalloc(const kvq_cache *cache, int32_t layer, const void *K, const void *V,
                                   const void *Q, const int32_t *ctx_len, float scale, float *out,
                                   int32_t n_splits, void *stream)
{
    if (!K || !V || !aligned16(K) || !aligned16(V))
        return KVQ_E_ARG;
    return attn_decode(cache, layer, K, V, Q, ctx_len, scale, out, nullptr, 0, n_splits, stream, true);
}

int kvq_attn_prefill_chunk(const kvq_cache *cache, int32_t layer, const void *Q, int32_t n_tok,
                           const int32_t *q_pos0, float scale, float *out, void *stream)
{
    int rc = check_layer(cache, layer);
    if (rc)
        return rc;
    const kvq_shape &sh = cache->shape;
    if (!Q || !q_pos0 || !out || !aligned16(Q) || !aligned16(out))
        return KVQ_E_ARG;
    if (!isfinite(scale))
        return KVQ_E_ARG;
    if (n_tok < 1)
        return KVQ_E_RANGE;
    for (int s = 0; s < sh.n_seqs; s++)
        if (q_pos0[s] < 0 || (int64_t)q_pos0[s] + n_tok > sh.max_ctx)
            return KVQ_E_RANGE;

    const kvq_plane &kp = cache->k[layer], &vp = cache->v[layer];
    PrefillArgs a;
    memset(&a, 0, sizeof(a));
    a.kc = (const uint8_t *)kp.codes;
    a.ks = (const uint16_t *)kp.scales;
    a.vc = (const uint8_t *)vp.codes;
    a.vs = (const uint16_t *)vp.scales;
    a.kqh = high_bits(sh, kp);
    a.vqh = high_bits(sh, vp);
    a.q = (const uint16_t *)Q;
    a.out = out;
    a.Hq = sh.n_q_heads;
    a.Hkv = sh.n_kv_heads;
    a.G = sh.n_q_heads / sh.n_kv_heads;
    a.Tc = (int32_t)capacity(sh.max_ctx);
    a.n_tok = n_tok;
    a.n_seqs = sh.n_seqs;
    while ((1 << a.gp_log2) < a.G)
        a.gp_log2++;
    a.c2 = (float)((double)scale * 1.4426950408889634);
    memcpy(a.q_pos0, q_pos0, sizeof(int32_t) * sh.n_seqs);
    hipError_t e = launch_prefill(kp.type, vp.type, sh.head_dim, a, (hipStream_t)stream);
    return e == hipSuccess ? KVQ_OK : KVQ_E_HIP;
}

}  // extern "C"
