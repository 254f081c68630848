/* Drives every entry point of the CPU oracle on small ragged shapes, for a
 * build under AddressSanitizer and UndefinedBehaviorSanitizer (see
 * tests/test_oracle_sanitize.py).  The oracle source is compiled into this
 * program; nothing here checks values (the other oracle tests do): the run
 * passes when no sanitizer reports an error. */
#include "../../oracle/moe_q4_oracle.c"

#include <stdio.h>

static uint64_t lcg_state = 88172645463325252ull;
static float lcg_normalish(void)   /* a sum of uniforms, centred: enough for shapes of data */
{
    float s = 0.0f;
    for (int i = 0; i < 4; i++) {
        lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
        s += (float)((lcg_state >> 40) & 0xffffff) / 16777216.0f;
    }
    return s - 2.0f;
}

static float *fill(int64_t n, float scale)
{
    float *p = (float *)malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; i++) p[i] = lcg_normalish() * scale;
    return p;
}

static void run_layer(int64_t H, int64_t I, int64_t E, int32_t k, int32_t shared, int32_t wfmt, int bias)
{
    const int64_t T = 7, S = shared ? 1 : 0;
    size_t (*row_bytes)(int64_t) = wfmt ? orc_q8w_row_bytes : orc_q4_row_bytes;
    void (*pack)(const float *, int64_t, int64_t, uint8_t *) = wfmt ? orc_q8w_pack : orc_q4_pack;
    float *wr = fill(H * E, 0.02f), *b = bias ? fill(E, 1.0f) : NULL;
    float *wg = fill(E * I * H, 0.02f), *wu = fill(E * I * H, 0.02f), *wd = fill(E * H * I, 0.02f);
    float *sg = fill(I * H, 0.02f), *su = fill(I * H, 0.02f), *sd = fill(H * I, 0.02f);
    uint8_t *g = malloc((size_t)(E * I) * row_bytes(H)), *u = malloc((size_t)(E * I) * row_bytes(H));
    uint8_t *d = malloc((size_t)(E * H) * row_bytes(I));
    uint8_t *pg = malloc((size_t)I * row_bytes(H)), *pu = malloc((size_t)I * row_bytes(H));
    uint8_t *pd = malloc((size_t)H * row_bytes(I));
    pack(wg, E * I, H, g); pack(wu, E * I, H, u); pack(wd, E * H, I, d);
    pack(sg, I, H, pg); pack(su, I, H, pu); pack(sd, H, I, pd);
    orc_layer L = {H, I, E, k, shared, wr, b, g, u, d, shared ? pg : NULL, shared ? pu : NULL,
                   shared ? pd : NULL, wfmt};
    float *x = fill(T * H, 1.0f);
    if (!wfmt) {
        float *logits = malloc((size_t)(T * E) * sizeof(float));
        int32_t *ids = malloc((size_t)(T * k) * sizeof(int32_t));
        float *w32 = malloc((size_t)(T * k) * sizeof(float));
        double *w64 = malloc((size_t)(T * k) * sizeof(double));
        int32_t *counts = malloc((size_t)E * sizeof(int32_t)), *offsets = malloc((size_t)(E + 1) * sizeof(int32_t));
        int32_t *perm = malloc((size_t)(T * k) * sizeof(int32_t)), *inv = malloc((size_t)(T * k) * sizeof(int32_t));
        orc_router_logits(x, T, H, wr, E, b, logits);
        for (int64_t e = 0; e < E; e++) logits[e] = 0.5f;        /* an all-tied token */
        orc_topk(logits, T, E, k, ids, w32, w64);
        orc_route_permutation(ids, T, k, E, counts, offsets, perm, inv);
        int64_t toks[3] = {0, 3, T - 1};
        double *y = malloc((size_t)(3 * H) * sizeof(double));
        orc_prefill_ref(&L, x, ids, w64, toks, 3, y);
        float *deq = malloc((size_t)(I * H) * sizeof(float));
        orc_q4_dequant(pg, I, H, deq);
        free(logits); free(ids); free(w32); free(w64); free(counts); free(offsets); free(perm); free(inv);
        free(y); free(deq);
    } else {
        float *deq = malloc((size_t)(I * H) * sizeof(float));
        orc_q8w_dequant(pg, I, H, deq);
        free(deq);
    }
    /* decode with the full trace, then without */
    float *yd = malloc((size_t)H * sizeof(float));
    orc_decode_trace tr;
    tr.logits = malloc((size_t)E * sizeof(float)); tr.ids = malloc((size_t)k * sizeof(int32_t));
    tr.w = malloc((size_t)k * sizeof(float)); tr.qx = malloc((size_t)H); tr.dx = malloc((size_t)(H / 32) * sizeof(float));
    tr.gate = malloc((size_t)((k + S) * I) * sizeof(float)); tr.up = malloc((size_t)((k + S) * I) * sizeof(float));
    tr.qh = malloc((size_t)((k + S) * I)); tr.dh = malloc((size_t)((k + S) * (I / 32)) * sizeof(float));
    tr.o = malloc((size_t)((k + S) * H) * sizeof(float));
    orc_decode(&L, x, yd, &tr);
    orc_decode(&L, x + H, yd, NULL);
    /* the W4A8 / W8A8 row program with the dots export */
    int8_t *qa = malloc((size_t)H); float *da = malloc((size_t)(H / 32) * sizeof(float));
    int32_t *dots = malloc((size_t)(I * (H / 32)) * sizeof(int32_t)); float *out = malloc((size_t)I * sizeof(float));
    orc_q8_quantize(x, 1, H, qa, da);
    if (wfmt) orc_w8a8_gemv(pg, I, H, qa, da, dots, out);
    else orc_w4a8_gemv(pg, I, H, qa, da, dots, out);
    float *yn = malloc((size_t)(T * H) * sizeof(float));
    orc_rmsnorm(x, T, H, 1e-6f, yn);
    free(yd); free(tr.logits); free(tr.ids); free(tr.w); free(tr.qx); free(tr.dx); free(tr.gate); free(tr.up);
    free(tr.qh); free(tr.dh); free(tr.o); free(qa); free(da); free(dots); free(out); free(yn);
    free(wr); free(b); free(wg); free(wu); free(wd); free(sg); free(su); free(sd);
    free(g); free(u); free(d); free(pg); free(pu); free(pd); free(x);
}

int main(void)
{
    /* scalar helpers on edge values: fp16 subnormals, overflow, zeros; the
     * fixed exp and silu at their clamps */
    const float f[] = {0.0f, -0.0f, 1e-8f, -6.1e-5f, 65504.0f, 70000.0f, 1e-30f, 3.0f};
    for (unsigned i = 0; i < sizeof f / sizeof f[0]; i++) (void)orc_f16_to_f32(orc_f32_to_f16(f[i]));
    const float xe[] = {-1000.0f, -104.0f, -20.0f, 0.0f, 20.0f, 89.0f, 1000.0f};
    for (unsigned i = 0; i < sizeof xe / sizeof xe[0]; i++) { (void)orc_exp_p(xe[i]); (void)orc_silu_p(xe[i]); }
    float v[5] = {1, 2, 3, 4, 5};
    (void)orc_tree_sum(v, 5);
    (void)orc_tree_sum(v, 1);
    /* a zero block and an fp16-subnormal scale through both packers */
    float w[64] = {0};
    for (int i = 32; i < 64; i++) w[i] = 1e-7f * (float)(i - 40);
    uint8_t q4[36], q8[68];
    orc_q4_pack(w, 1, 64, q4);
    orc_q8w_pack(w, 1, 64, q8);
    /* layers: ragged chunk counts, k = E, E = 1, bias, no shared expert, Q8_0 */
    run_layer(96, 64, 5, 2, 1, 0, 1);
    run_layer(256, 128, 8, 8, 0, 0, 0);
    run_layer(64, 32, 1, 1, 1, 0, 0);
    run_layer(160, 96, 6, 3, 1, 1, 1);
    printf("oracle driver: OK\n");
    return 0;
}
