/*
 * kvq_oracle.c -- plain, slow CPU oracle for the mixed-precision quantized
 * KV cache (keys and values stored at independently chosen precisions) and
 * for attention decode / causal chunked prefill over it.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load this
 * library: only the tests, the package's smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source with the HIP library; the
 * storage layout it writes is re-derived here from the written contract.
 *
 * Sources (all of them web pages; cited by title and section):
 *   [KVSplit]  "KVSplit - 2- bis 3-mal laengerer Kontext auf Apple Silicon"
 *              (news.hada.io topic 20969): sections "Zentrale Benchmark-
 *              Ergebnisse", "Vergleich der Speicherersparnis",
 *              "Wissenschaftliche Einsichten und Versuchsergebnisse".
 *   [Tokios]   "llama.cpp fuer Geschwindigkeit und Speicher optimieren"
 *              (docs.tokios.com): sections "Flash Attention",
 *              "KV-Cache-Praezision", "Batch-Groessen-Abstimmung".
 *   [Issue]    llama.cpp issue "Eval bug: Metal fails mixed quantized KV on
 *              Apple Silicon when Flash Attention is unavailable ...":
 *              the llama_kv_cache size lines under "Relevant log output".
 *
 * What the pages fix, and the readings taken where they are silent:
 *   - Cache types f16 / q8_0 / q4_0, chosen independently for K and V
 *     ([Tokios] KV-Cache-Praezision table and the sentence that keys and
 *     values can be set independently; [KVSplit] K8V4 / K4V4 configs).
 *   - q8_0 and q4_0 are llama.cpp's (ggml) 32-element block formats with a
 *     binary16 scale per block: 34 and 18 bytes per 32 elements.  The byte
 *     totals printed on [KVSplit] (Vergleich der Speicherersparnis) and in
 *     [Issue] (llama_kv_cache lines) hold exactly under that size, and the
 *     byte-count tests pin it.
 *   - q8_0: d = amax/127, codes = round(x/d) in [-127,127].
 *     q4_0: d = (signed value of largest magnitude)/(-8),
 *           code = clamp(trunc(x/d + 8.5), 0, 15), two codes per byte.
 *     Op-level reading (both sides follow it bit for bit): d is computed in
 *     binary32, rounded once to binary16 (round to nearest even); codes are
 *     taken against the STORED binary16 scale through its binary32
 *     reciprocal; q8_0 rounds half away from zero; q4_0 rounds x*id and
 *     then adds 8.5 (two roundings, no fused multiply-add); the q4_0 signed
 *     maximum takes the lowest index among equal magnitudes and is +0 for an
 *     all-zero block; a zero stored scale gives reciprocal 0; codes are
 *     clamped to their ranges (only reachable with subnormal scales).
 *     Nibble order: byte i of a block holds element i (low nibble) and
 *     element i+16 (high nibble).
 *   - q5_0 (a fourth type; the pages only name it: a comment in [Issue]'s
 *     thread reports q5_0/q5_0 as the working middle ground): ggml's 5-bit
 *     32-element block, read the way q4_0 is read above with the
 *     5-bit range: d = (signed value of largest magnitude)/(-16),
 *     code = clamp(trunc(x*id + 16.5), 0, 31), value d*(code - 16); 22 bytes
 *     per 32 elements (16 bytes of low nibbles in q4_0's order, 32 high bits,
 *     the binary16 scale).  Parity with llama.cpp's own q5_0 is unpinned.
 *   - turbo3 (values only): the page "Benchmark TurboQuant en Apple
 *     Silicon" (section "Que es TurboQuant?") names a random rotation by the
 *     Walsh-Hadamard transform to make the data Gaussian, an optimal scalar
 *     quantizer, 3 bits per value, keys kept at q8_0.  Nothing more of the
 *     format is on the page; the reading taken, per 32-element block:
 *       y = H * (s . x), H the 32x32 Sylvester Hadamard matrix
 *         (H[k][i] = (-1)^popcount(k & i)), s_i = -1 where bit i of
 *         TQ3_SIGNS is set; computed in binary64, which is exact here
 *         (binary16 inputs: every partial sum is a multiple of 2^-24 below
 *         2^21);
 *       codebook: the 8 Lloyd-Max levels of N(0,1), rounded to binary16;
 *       d = f16(f32(max_k |y_k|) / L_7) (the block maximum lands on the
 *         outermost level), id = d ? 1/d : 0;
 *       code_k = number of midpoints (L_j + L_j+1)/2 that f32(y_k) * id
 *         reaches (>=), so the nearest level, 0..7;
 *       value: x^ = (1/32) * s . (H * (d * L[code])).
 *     Stored as a 2-bit plane (byte j of a block: elements j, j+8, j+16,
 *     j+24 at bits 0, 2, 4, 6) and a 32-bit word of the codes' third bits
 *     (bit i = element i): 14 bytes per 32 elements with the scale.
 *   - Attention: flash attention is exactly standard softmax attention
 *     ([Tokios] Flash Attention: mathematically equivalent, no
 *     approximation), so decode is textbook softmax attention over the
 *     dequantized cache, here in binary64.
 *   - Chunked prefill ([Tokios] Batch-Groessen-Abstimmung: the prompt is
 *     processed in micro-batches): query i of a chunk at position p0+i
 *     attends to cache positions 0..p0+i.
 *   - GQA: query head hq reads kv head hq / (n_q_heads / n_kv_heads).
 *
 * Storage layout (the library's written contract, re-implemented here):
 *   Tc = max_ctx rounded up to a multiple of 32; nb = head_dim/32;
 *   row code bytes R = 2*D (f16), D (q8_0), D/2 (q4_0 and the q5_0 nibbles).
 *   K plane, token-major:  code byte r of token t of (s,h) at
 *       ((s*H + h)*Tc + t)*R + r;  scale of block b at ((s*H+h)*Tc + t)*nb + b.
 *   V plane, 8-token interleaved: with unit size w = 2 (f16) or 1 byte,
 *       U = R/w units per row, unit u of token t at unit index
 *       (((s*H + h)*(Tc/8) + t/8)*U + u)*8 + t%8;
 *       scale of block b at (((s*H + h)*(Tc/8) + t/8)*nb + b)*8 + t%8.
 *   turbo3: row code bytes R = D/4 (the 2-bit planes), then the third-bit
 *   words exactly as q5_0's high-bit words below.
 *   q5_0: the code stream holds the nibble rows exactly as q4_0 does, then,
 *   from byte S*H*Tc*R on, one little-endian 32-bit word of high bits per
 *   (token, block), indexed like that block's scale (bit i = bit 4 of the
 *   code of element i).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KVQO_F16 0
#define KVQO_Q8_0 1
#define KVQO_Q4_0 2
#define KVQO_Q5_0 3
#define KVQO_TQ3 4

/* turbo3: rotation signs and the binary16 bits of the Lloyd-Max levels of
 * N(0,1) for 8 levels (+-0.2451, +-0.7560, +-1.3439, +-2.1519 rounded). */
#define TQ3_SIGNS 0x9E3779B9u
static const uint16_t TQ3_LEVELS[8] = {0xC04E, 0xBD60, 0xBA0C, 0xB3D8, 0x33D8, 0x3A0C, 0x3D60, 0x404E};
#define KVQO_ROLE_K 0
#define KVQO_ROLE_V 1

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32, written from the format definition. */
/* ------------------------------------------------------------------ */

float kvqo_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* zero / subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return (float)(sign ? -v : v);
}

/* Round to nearest, ties to even. */
uint16_t kvqo_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7e00);
    if (isinf(f))
        return (uint16_t)(sign | 0x7c00); /* infinities stay infinite */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: integer multiple of 2^-24 (1024 means 2^-14) */
        double n = nearbyint(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int ex;
    frexp(a, &ex); /* a = fr * 2^ex, fr in [0.5,1)  =>  2^(ex-1) <= a */
    int e = ex - 1;
    double n = nearbyint(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (n >= 2048.0) {
        n = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)n - 1024));
}

void kvqo_f32_to_f16_n(const float *x, uint16_t *y, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        y[i] = kvqo_f32_to_f16(x[i]);
}

void kvqo_f16_to_f32_n(const uint16_t *x, float *y, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        y[i] = kvqo_f16_to_f32(x[i]);
}

/* ------------------------------------------------------------------ */
/* Block quantizers (32 elements, binary16 scale).                     */
/* ------------------------------------------------------------------ */

static float round_half_away(float v) { return roundf(v); } /* C roundf */

void kvqo_quantize_q8_0(const uint16_t *x16, uint16_t *d_out, int8_t *q)
{
    float x[32];
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
        x[i] = kvqo_f16_to_f32(x16[i]);
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    float d32 = amax / 127.0f;
    uint16_t d16 = kvqo_f32_to_f16(d32);
    float d = kvqo_f16_to_f32(d16);
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    for (int i = 0; i < 32; i++) {
        float v = x[i] * id;
        float r = round_half_away(v);
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        q[i] = (int8_t)r;
    }
    *d_out = d16;
}

void kvqo_quantize_q4_0(const uint16_t *x16, uint16_t *d_out, uint8_t *packed)
{
    float x[32];
    float amax = 0.0f;
    float m = 0.0f; /* +0 unless some |x_i| > 0 */
    for (int i = 0; i < 32; i++) {
        x[i] = kvqo_f16_to_f32(x16[i]);
        float a = fabsf(x[i]);
        if (a > amax) { /* strict: the lowest index wins a tie */
            amax = a;
            m = x[i];
        }
    }
    float d32 = m / -8.0f;
    uint16_t d16 = kvqo_f32_to_f16(d32);
    float d = kvqo_f16_to_f32(d16);
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    int c[32];
    for (int i = 0; i < 32; i++) {
        float t = x[i] * id;
        float u = t + 8.5f;
        int ci = (int)truncf(u);
        if (ci > 15)
            ci = 15;
        if (ci < 0)
            ci = 0;
        c[i] = ci;
    }
    for (int i = 0; i < 16; i++)
        packed[i] = (uint8_t)(c[i] | (c[i + 16] << 4));
    *d_out = d16;
}

/* q5_0: as q4_0 with 32 levels.  Output: 16 nibble bytes (element i low,
 * i+16 high, low 4 bits of each code) and the 32 high bits in *qh. */
void kvqo_quantize_q5_0(const uint16_t *x16, uint16_t *d_out, uint8_t *packed, uint32_t *qh)
{
    float x[32];
    float amax = 0.0f;
    float m = 0.0f; /* +0 unless some |x_i| > 0 */
    for (int i = 0; i < 32; i++) {
        x[i] = kvqo_f16_to_f32(x16[i]);
        float a = fabsf(x[i]);
        if (a > amax) { /* strict: the lowest index wins a tie */
            amax = a;
            m = x[i];
        }
    }
    float d32 = m / -16.0f;
    uint16_t d16 = kvqo_f32_to_f16(d32);
    float d = kvqo_f16_to_f32(d16);
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    int c[32];
    for (int i = 0; i < 32; i++) {
        float t = x[i] * id;
        float u = t + 16.5f;
        int ci = (int)truncf(u);
        if (ci > 31)
            ci = 31;
        if (ci < 0)
            ci = 0;
        c[i] = ci;
    }
    uint32_t h = 0;
    for (int i = 0; i < 16; i++)
        packed[i] = (uint8_t)((c[i] & 15) | ((c[i + 16] & 15) << 4));
    for (int i = 0; i < 32; i++)
        h |= (uint32_t)(c[i] >> 4) << i;
    *qh = h;
    *d_out = d16;
}

/* The 32-point Walsh-Hadamard transform in Sylvester order, in place,
 * butterflies of span 1, 2, 4, 8, 16 (binary64). */
static void wht32(double *v)
{
    for (int len = 1; len < 32; len <<= 1)
        for (int i = 0; i < 32; i += 2 * len)
            for (int k = i; k < i + len; k++) {
                double a = v[k], b = v[k + len];
                v[k] = a + b;
                v[k + len] = a - b;
            }
}

/* exported for the tests: out = H * in (binary64) */
void kvqo_wht32(const double *in, double *out)
{
    memcpy(out, in, 32 * sizeof(double));
    wht32(out);
}

/* turbo3 block: 8 bytes of 2-bit planes + 4 bytes (little-endian) of third bits. */
void kvqo_quantize_tq3(const uint16_t *x16, uint16_t *d_out, uint8_t *packed)
{
    double y[32];
    for (int i = 0; i < 32; i++) {
        double x = (double)kvqo_f16_to_f32(x16[i]);
        y[i] = ((TQ3_SIGNS >> i) & 1u) ? -x : x;
    }
    wht32(y);
    double m = 0.0;
    for (int k = 0; k < 32; k++)
        if (fabs(y[k]) > m)
            m = fabs(y[k]);
    float lmax = kvqo_f16_to_f32(TQ3_LEVELS[7]);
    float d32 = (float)m / lmax;
    uint16_t d16 = kvqo_f32_to_f16(d32);
    float d = kvqo_f16_to_f32(d16);
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    float mid[7];
    for (int j = 0; j < 7; j++)
        mid[j] = (kvqo_f16_to_f32(TQ3_LEVELS[j]) + kvqo_f16_to_f32(TQ3_LEVELS[j + 1])) * 0.5f; /* exact */
    memset(packed, 0, 12);
    uint32_t hi = 0;
    for (int k = 0; k < 32; k++) {
        float t = (float)y[k] * id;
        int c = 0;
        for (int j = 0; j < 7; j++)
            c += (t >= mid[j]);
        packed[k % 8] |= (uint8_t)((c & 3) << (2 * (k / 8)));
        hi |= (uint32_t)(c >> 2) << k;
    }
    for (int b = 0; b < 4; b++)
        packed[8 + b] = (uint8_t)(hi >> (8 * b));
    *d_out = d16;
}

/* f16 "quantizer": the block is stored as is. */
static void store_f16_block(const uint16_t *x16, uint8_t *codes)
{
    memcpy(codes, x16, 64);
}

int kvqo_block_code_bytes(int type)
{
    /* q5_0: 16 nibble bytes, then the 32 high bits as 4 little-endian bytes;
     * turbo3: 8 bytes of 2-bit planes, then the 32 third bits */
    return type == KVQO_F16 ? 64 : type == KVQO_Q8_0 ? 32 : type == KVQO_Q4_0 ? 16 : type == KVQO_Q5_0 ? 20
         : type == KVQO_TQ3 ? 12 : -1;
}

/* Contiguous blocks: x [n][32] -> codes [n][block_code_bytes], d [n]. */
void kvqo_quantize_blocks(int type, const uint16_t *x, int64_t n, uint16_t *d, uint8_t *codes)
{
    int cb = kvqo_block_code_bytes(type);
    for (int64_t i = 0; i < n; i++) {
        if (type == KVQO_Q8_0)
            kvqo_quantize_q8_0(x + 32 * i, d + i, (int8_t *)(codes + cb * i));
        else if (type == KVQO_Q4_0)
            kvqo_quantize_q4_0(x + 32 * i, d + i, codes + cb * i);
        else if (type == KVQO_Q5_0) {
            uint32_t qh = 0;
            kvqo_quantize_q5_0(x + 32 * i, d + i, codes + cb * i, &qh);
            for (int k = 0; k < 4; k++)
                codes[cb * i + 16 + k] = (uint8_t)(qh >> (8 * k));
        } else if (type == KVQO_TQ3) {
            kvqo_quantize_tq3(x + 32 * i, d + i, codes + cb * i);
        } else {
            store_f16_block(x + 32 * i, codes + cb * i);
            d[i] = 0;
        }
    }
}

/* Dequantized value of element e of a block, in binary64 (exact). */
static double dequant_elem(int type, uint16_t d16, const uint8_t *bc, int e)
{
    if (type == KVQO_F16) {
        uint16_t h = (uint16_t)(bc[2 * e] | (bc[2 * e + 1] << 8));
        return (double)kvqo_f16_to_f32(h);
    }
    double d = (double)kvqo_f16_to_f32(d16);
    if (type == KVQO_Q8_0)
        return d * (double)(int8_t)bc[e];
    int c = (e < 16) ? (bc[e] & 0x0f) : (bc[e - 16] >> 4);
    if (type == KVQO_Q4_0)
        return d * (double)(c - 8);
    /* q5_0: bit e of the little-endian word at bytes 16..19 is bit 4 */
    c |= ((bc[16 + e / 8] >> (e % 8)) & 1) << 4;
    return d * (double)(c - 16);
}

/* turbo3: the whole block (the rotation mixes its elements), binary64. */
static void dequant_tq3(uint16_t d16, const uint8_t *bc, double *out)
{
    double d = (double)kvqo_f16_to_f32(d16);
    uint32_t hi = (uint32_t)bc[8] | ((uint32_t)bc[9] << 8) | ((uint32_t)bc[10] << 16) | ((uint32_t)bc[11] << 24);
    double y[32];
    for (int k = 0; k < 32; k++) {
        int c = ((bc[k % 8] >> (2 * (k / 8))) & 3) | (int)(((hi >> k) & 1u) << 2);
        y[k] = d * (double)kvqo_f16_to_f32(TQ3_LEVELS[c]);
    }
    wht32(y); /* H is symmetric and H*H = 32 I */
    for (int i = 0; i < 32; i++)
        out[i] = (((TQ3_SIGNS >> i) & 1u) ? -y[i] : y[i]) / 32.0;
}

static void dequant_block(int type, uint16_t d16, const uint8_t *bc, double *out)
{
    if (type == KVQO_TQ3) {
        dequant_tq3(d16, bc, out);
        return;
    }
    for (int e = 0; e < 32; e++)
        out[e] = dequant_elem(type, d16, bc, e);
}

void kvqo_dequantize_blocks(int type, const uint16_t *d, const uint8_t *codes, int64_t n, double *out)
{
    int cb = kvqo_block_code_bytes(type);
    for (int64_t i = 0; i < n; i++)
        dequant_block(type, d[i], codes + cb * i, out + 32 * i);
}

/* ------------------------------------------------------------------ */
/* Plane layout and byte accounting.                                    */
/* ------------------------------------------------------------------ */

typedef struct {
    int32_t type;
    int32_t role;
    uint8_t *codes;
    uint16_t *scales; /* NULL for f16 */
} kvqo_plane;

typedef struct {
    int32_t n_seqs, n_q_heads, n_kv_heads, head_dim, max_ctx;
} kvqo_shape;

int64_t kvqo_capacity(int64_t max_ctx) { return (max_ctx + 31) / 32 * 32; }

int64_t kvqo_row_code_bytes(int type, int64_t D)
{
    /* q5_0: nibble rows; turbo3: 2-bit plane rows */
    return type == KVQO_F16 ? 2 * D : type == KVQO_Q8_0 ? D : type == KVQO_TQ3 ? D / 4 : D / 2;
}

/* Types whose code stream continues with one 32-bit word per (row, block). */
static int has_bit_words(int type) { return type == KVQO_Q5_0 || type == KVQO_TQ3; }

void kvqo_plane_bytes(int type, int64_t n_seqs, int64_t n_kv_heads, int64_t head_dim, int64_t max_ctx,
                      int64_t *codes_bytes, int64_t *scale_bytes)
{
    int64_t rows = n_seqs * n_kv_heads * kvqo_capacity(max_ctx);
    *codes_bytes = rows * kvqo_row_code_bytes(type, head_dim);
    if (has_bit_words(type))
        *codes_bytes += rows * (head_dim / 32) * 4; /* the high-bit words */
    *scale_bytes = (type == KVQO_F16) ? 0 : rows * (head_dim / 32) * 2;
}

/* Byte address of code byte r (0 <= r < R) of token t of pair (s,h). */
static int64_t code_byte_addr(const kvqo_plane *p, const kvqo_shape *sh, int s, int h, int64_t t, int64_t r)
{
    int64_t Tc = kvqo_capacity(sh->max_ctx);
    int64_t R = kvqo_row_code_bytes(p->type, sh->head_dim);
    int64_t pair = (int64_t)s * sh->n_kv_heads + h;
    if (p->role == KVQO_ROLE_K)
        return (pair * Tc + t) * R + r;
    int64_t w = (p->type == KVQO_F16) ? 2 : 1;
    int64_t U = R / w;
    int64_t u = r / w;
    int64_t unit = ((pair * (Tc / 8) + t / 8) * U + u) * 8 + t % 8;
    return unit * w + r % w;
}

static int64_t scale_index(const kvqo_plane *p, const kvqo_shape *sh, int s, int h, int64_t t, int b)
{
    int64_t Tc = kvqo_capacity(sh->max_ctx);
    int64_t nb = sh->head_dim / 32;
    int64_t pair = (int64_t)s * sh->n_kv_heads + h;
    if (p->role == KVQO_ROLE_K)
        return (pair * Tc + t) * nb + b;
    return ((pair * (Tc / 8) + t / 8) * nb + b) * 8 + t % 8;
}

/* q5_0: byte address of the first byte of the high-bit word of block b of
 * token t of pair (s,h): after all nibble rows, indexed like the scale. */
static int64_t qh_byte_addr(const kvqo_plane *p, const kvqo_shape *sh, int s, int h, int64_t t, int b)
{
    int64_t rows = (int64_t)sh->n_seqs * sh->n_kv_heads * kvqo_capacity(sh->max_ctx);
    return rows * kvqo_row_code_bytes(p->type, sh->head_dim) + 4 * scale_index(p, sh, s, h, t, b);
}

/* Quantize new rows x [S][n_new][H][D] (binary16 bits) into positions
 * pos[s] .. pos[s]+n_new-1 of plane p.  Caller guarantees the range. */
void kvqo_append(const kvqo_plane *p, const kvqo_shape *sh, const uint16_t *x, int n_new, const int32_t *pos)
{
    int S = sh->n_seqs, H = sh->n_kv_heads, D = sh->head_dim, nb = D / 32;
    int cb = kvqo_block_code_bytes(p->type);
#pragma omp parallel for collapse(2) schedule(static)
    for (int s = 0; s < S; s++)
        for (int i = 0; i < n_new; i++) {
            for (int h = 0; h < H; h++) {
                int64_t t = (int64_t)pos[s] + i;
                const uint16_t *row = x + (((int64_t)s * n_new + i) * H + h) * D;
                for (int b = 0; b < nb; b++) {
                    uint8_t bc[64];
                    uint16_t d16 = 0;
                    kvqo_quantize_blocks(p->type, row + 32 * b, 1, &d16, bc);
                    int nib = has_bit_words(p->type) ? cb - 4 : cb; /* bytes that live in the rows */
                    for (int r = 0; r < nib; r++)
                        p->codes[code_byte_addr(p, sh, s, h, t, (int64_t)b * nib + r)] = bc[r];
                    if (has_bit_words(p->type))
                        for (int k = 0; k < 4; k++)
                            p->codes[qh_byte_addr(p, sh, s, h, t, b) + k] = bc[nib + k];
                    if (p->type != KVQO_F16)
                        p->scales[scale_index(p, sh, s, h, t, b)] = d16;
                }
            }
        }
}

/* Dequantized rows t0..t0+n-1 of pair (s,h) into out [n][D] (binary64). */
void kvqo_read_rows(const kvqo_plane *p, const kvqo_shape *sh, int s, int h, int64_t t0, int64_t n, double *out)
{
    int D = sh->head_dim, nb = D / 32;
    int cb = kvqo_block_code_bytes(p->type);
    for (int64_t k = 0; k < n; k++) {
        int64_t t = t0 + k;
        for (int b = 0; b < nb; b++) {
            uint8_t bc[64];
            int nib = has_bit_words(p->type) ? cb - 4 : cb;
            for (int r = 0; r < nib; r++)
                bc[r] = p->codes[code_byte_addr(p, sh, s, h, t, (int64_t)b * nib + r)];
            if (has_bit_words(p->type))
                for (int k = 0; k < 4; k++)
                    bc[nib + k] = p->codes[qh_byte_addr(p, sh, s, h, t, b) + k];
            uint16_t d16 = (p->type == KVQO_F16) ? 0 : p->scales[scale_index(p, sh, s, h, t, b)];
            dequant_block(p->type, d16, bc, out + k * D + 32 * b);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Attention in binary64.                                               */
/* ------------------------------------------------------------------ */

/* Textbook softmax attention of one query q[D] over rows 0..ctx-1 of the
 * dequantized keys Kd / values Vd ([*][D]).  scores: scratch [ctx]. */
static void softmax_attend(const double *q, const double *Kd, const double *Vd, int64_t ctx, int D, double scale,
                           double *scores, double *out)
{
    double mx = -INFINITY;
    for (int64_t t = 0; t < ctx; t++) {
        double acc = 0.0;
        for (int c = 0; c < D; c++)
            acc += q[c] * Kd[t * D + c];
        scores[t] = scale * acc;
        if (scores[t] > mx)
            mx = scores[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < ctx; t++) {
        scores[t] = exp(scores[t] - mx);
        l += scores[t];
    }
    for (int c = 0; c < D; c++)
        out[c] = 0.0;
    for (int64_t t = 0; t < ctx; t++) {
        double w = scores[t] / l;
        for (int c = 0; c < D; c++)
            out[c] += w * Vd[t * D + c];
    }
}

/* Decode: Q [S][Hq][D] (binary16 bits), ctx_len[S]; out [S][Hq][D].
 * want: optional mask [S][Hq] selecting the outputs to compute. */
void kvqo_attn_decode(const kvqo_plane *kp, const kvqo_plane *vp, const kvqo_shape *sh, const uint16_t *Q,
                      const int32_t *ctx_len, double scale, const uint8_t *want, double *out)
{
    int S = sh->n_seqs, Hq = sh->n_q_heads, H = sh->n_kv_heads, D = sh->head_dim;
    int G = Hq / H;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < S; s++)
        for (int h = 0; h < H; h++) {
            int any = 0;
            for (int g = 0; g < G; g++)
                any |= want == NULL || want[s * Hq + h * G + g];
            if (!any)
                continue;
            int64_t ctx = ctx_len[s];
            double *Kd = malloc(sizeof(double) * ctx * D);
            double *Vd = malloc(sizeof(double) * ctx * D);
            double *sc = malloc(sizeof(double) * ctx);
            double *q = malloc(sizeof(double) * D);
            kvqo_read_rows(kp, sh, s, h, 0, ctx, Kd);
            kvqo_read_rows(vp, sh, s, h, 0, ctx, Vd);
            for (int g = 0; g < G; g++) {
                int hq = h * G + g;
                if (want != NULL && !want[s * Hq + hq])
                    continue;
                for (int c = 0; c < D; c++)
                    q[c] = (double)kvqo_f16_to_f32(Q[((int64_t)s * Hq + hq) * D + c]);
                softmax_attend(q, Kd, Vd, ctx, D, scale, sc, out + ((int64_t)s * Hq + hq) * D);
            }
            free(Kd);
            free(Vd);
            free(sc);
            free(q);
        }
}

/* Causal chunked prefill: Q [S][n_tok][Hq][D]; query i of sequence s sits
 * at position q_pos0[s]+i and attends to positions 0..q_pos0[s]+i.
 * want: optional mask [S][n_tok][Hq]; out [S][n_tok][Hq][D]. */
void kvqo_attn_prefill(const kvqo_plane *kp, const kvqo_plane *vp, const kvqo_shape *sh, const uint16_t *Q,
                       int n_tok, const int32_t *q_pos0, double scale, const uint8_t *want, double *out)
{
    int S = sh->n_seqs, Hq = sh->n_q_heads, H = sh->n_kv_heads, D = sh->head_dim;
    int G = Hq / H;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < S; s++)
        for (int h = 0; h < H; h++) {
            int any = 0;
            for (int i = 0; i < n_tok; i++)
                for (int g = 0; g < G; g++)
                    any |= want == NULL || want[((int64_t)s * n_tok + i) * Hq + h * G + g];
            if (!any)
                continue;
            int64_t ctx_max = (int64_t)q_pos0[s] + n_tok;
            double *Kd = malloc(sizeof(double) * ctx_max * D);
            double *Vd = malloc(sizeof(double) * ctx_max * D);
            double *sc = malloc(sizeof(double) * ctx_max);
            double *q = malloc(sizeof(double) * D);
            kvqo_read_rows(kp, sh, s, h, 0, ctx_max, Kd);
            kvqo_read_rows(vp, sh, s, h, 0, ctx_max, Vd);
            for (int i = 0; i < n_tok; i++)
                for (int g = 0; g < G; g++) {
                    int hq = h * G + g;
                    int64_t o = ((int64_t)s * n_tok + i) * Hq + hq;
                    if (want != NULL && !want[o])
                        continue;
                    for (int c = 0; c < D; c++)
                        q[c] = (double)kvqo_f16_to_f32(Q[o * D + c]);
                    softmax_attend(q, Kd, Vd, (int64_t)q_pos0[s] + i + 1, D, scale, sc, out + o * D);
                }
            free(Kd);
            free(Vd);
            free(sc);
            free(q);
        }
}

int kvqo_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
