/*
 * Drives every exported function of the CPU oracle (oracle/kvq_oracle.c,
 * compiled into this same translation unit) on tiny shapes of every cache
 * type, for a build with AddressSanitizer and UndefinedBehaviorSanitizer.
 * Test infrastructure: tests/test_oracle_sanitized.py compiles and runs it
 * on the CPU.  Every buffer is malloc'ed at exactly the size the oracle's
 * own byte accounting gives, so that a read or write past a plane, a block
 * or a row is reported.  Exit status 0 when the run completes; a sanitizer
 * report aborts it (-fno-sanitize-recover).
 */
#include "../oracle/kvq_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    /* xorshift64*: only a source of varied test bits */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

/* a finite binary16 value of magnitude below about 64 */
static uint16_t rand_f16(void)
{
    uint16_t h = (uint16_t)(next_u32() & 0xffff);
    uint16_t e = (uint16_t)((h >> 10) & 0x1f);
    if (e > 20)
        h = (uint16_t)((h & 0x83ff) | (uint16_t)((e - 11) << 10));
    return h;
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void run_pair(int kt, int vt, int D)
{
    const int S = 2, Hq = 4, H = 2, T = 45; /* max_ctx not a multiple of 32 */
    kvqo_shape sh = {S, Hq, H, D, T};
    kvqo_plane p[2];
    int types[2] = {kt, vt};
    for (int role = 0; role < 2; role++) {
        int64_t cb = 0, sb = 0;
        kvqo_plane_bytes(types[role], S, H, D, T, &cb, &sb);
        p[role].type = types[role];
        p[role].role = role;
        p[role].codes = xmalloc((size_t)cb);
        memset(p[role].codes, 0, (size_t)cb);
        p[role].scales = sb ? xmalloc((size_t)sb) : NULL;
        if (sb)
            memset(p[role].scales, 0, (size_t)sb);
    }
    /* append in two ragged chunks: positions 0..29 and 30..44 */
    int32_t pos0[2] = {0, 0}, pos1[2] = {30, 30};
    for (int chunk = 0; chunk < 2; chunk++) {
        int n = chunk ? 15 : 30;
        size_t cnt = (size_t)S * n * H * D;
        uint16_t *x = xmalloc(cnt * 2);
        for (int role = 0; role < 2; role++) {
            for (size_t i = 0; i < cnt; i++)
                x[i] = rand_f16();
            kvqo_append(&p[role], &sh, x, n, chunk ? pos1 : pos0);
        }
        free(x);
    }
    /* decode with ragged contexts, every output and a masked subset */
    uint16_t *Q = xmalloc((size_t)S * Hq * D * 2);
    for (int i = 0; i < S * Hq * D; i++)
        Q[i] = rand_f16();
    int32_t ctx[2] = {45, 1};
    double *out = xmalloc(sizeof(double) * S * Hq * D);
    kvqo_attn_decode(&p[0], &p[1], &sh, Q, ctx, 0.125, NULL, out);
    uint8_t want[8] = {1, 0, 0, 1, 0, 1, 0, 0};
    kvqo_attn_decode(&p[0], &p[1], &sh, Q, ctx, 0.125, want, out);
    free(out);
    free(Q);
    /* causal prefill: a 7-query chunk at positions 38..44 and 0..6 */
    const int n_tok = 7;
    uint16_t *Qc = xmalloc((size_t)S * n_tok * Hq * D * 2);
    for (int i = 0; i < S * n_tok * Hq * D; i++)
        Qc[i] = rand_f16();
    int32_t q0[2] = {38, 0};
    double *outp = xmalloc(sizeof(double) * S * n_tok * Hq * D);
    kvqo_attn_prefill(&p[0], &p[1], &sh, Qc, n_tok, q0, 0.125, NULL, outp);
    free(outp);
    free(Qc);
    /* every row of every pair, read back */
    double *rows = xmalloc(sizeof(double) * T * D);
    for (int role = 0; role < 2; role++)
        for (int s = 0; s < S; s++)
            for (int h = 0; h < H; h++)
                kvqo_read_rows(&p[role], &sh, s, h, 0, T, rows);
    free(rows);
    for (int role = 0; role < 2; role++) {
        free(p[role].codes);
        free(p[role].scales);
    }
}

static void run_blocks(int type)
{
    const int n = 5;
    int cb = kvqo_block_code_bytes(type);
    uint16_t *x = xmalloc(sizeof(uint16_t) * 32 * n);
    for (int i = 0; i < 32 * n; i++)
        x[i] = rand_f16();
    for (int i = 0; i < 32; i++) /* one all-zero block, one of negative zeros */
        x[32 + i] = 0, x[64 + i] = 0x8000;
    uint16_t *d = xmalloc(sizeof(uint16_t) * n);
    uint8_t *codes = xmalloc((size_t)cb * n);
    double *back = xmalloc(sizeof(double) * 32 * n);
    kvqo_quantize_blocks(type, x, n, d, codes);
    kvqo_dequantize_blocks(type, d, codes, n, back);
    free(back);
    free(codes);
    free(d);
    free(x);
}

int main(void)
{
    static const int types[5] = {KVQO_F16, KVQO_Q8_0, KVQO_Q4_0, KVQO_Q5_0, KVQO_TQ3};
    /* binary16 <-> binary32 over every bit pattern */
    for (uint32_t h = 0; h < 65536; h++) {
        float f = kvqo_f16_to_f32((uint16_t)h);
        if (!isnan(f) && kvqo_f32_to_f16(f) != (uint16_t)h) {
            fprintf(stderr, "binary16 round trip failed at 0x%04x\n", h);
            return 1;
        }
    }
    float fx[4] = {65520.0f, -1e-9f, 3.0e-8f, 1.0f};
    uint16_t hx[4];
    float fb[4];
    kvqo_f32_to_f16_n(fx, hx, 4);
    kvqo_f16_to_f32_n(hx, fb, 4);
    double win[32], wout[32];
    for (int i = 0; i < 32; i++)
        win[i] = (double)(int)(next_u32() % 200) - 100.0;
    kvqo_wht32(win, wout);
    for (int t = 0; t < 5; t++)
        run_blocks(types[t]);
    for (int D = 64; D <= 128; D += 64)
        for (int k = 0; k < 4; k++) /* turbo3 stores values only */
            for (int v = 0; v < 5; v++)
                run_pair(types[k], types[v], D);
    if (kvqo_max_threads() < 1)
        return 1;
    printf("oracle sanitized run: ok\n");
    return 0;
}
