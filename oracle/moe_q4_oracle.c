/*
 * moe_q4_oracle.c -- CPU oracle for the Q4_0 Mixture-of-Experts expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source, header, table or constant
 * generator with the HIP path.
 *
 * Plain, single-threaded C99.  Build with  gcc -O2 -ffp-contract=off  (no
 * fast-math) so that every float operation below is exactly the IEEE
 * operation written: a*b+c is two roundings unless fmaf() is spelled out.
 *
 * Sources (the web pages describing the method; cited by title + section):
 *   [FERMI] "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU:
 *           Hand-Written 4-bit CUDA Inference for Fermi", technical summary
 *           page.  Methodology 1 (GPU prefill runs a grouped 4-bit GEMM for the
 *           MoE; CPU decode runs a W4A8 integer kernel built on pmaddubsw),
 *           Methodology 2 (group-wise symmetric 4-bit weights of the Q4_0
 *           family, 8-bit activations on the decode path), Results (the thin-M
 *           GEMM is the structural bottleneck).
 *   [COMP]  "A Modern Multimodal Assistant on a 6 GB 2011 GPU: Stage-Validated,
 *           All-GPU CUDA Inference for Fermi", abstract (stage-wise validation
 *           against a locally generated reference; tie-breaking in index
 *           arithmetic must be pinned, not left to the implementation).
 *
 * The pages fix the *kind* of computation (Q4_0 group quantisation, W4A8
 * decode, routed experts) but no block size, scale rule, nibble order,
 * rounding, router, FFN form or float program.  The library fixes those as
 * follows, and this file is the plain statement of them:
 *   - Q4_0 block: 32 consecutive K-elements; fp16 scale d = fp16(amax/7);
 *     q = clamp(roundf(w/d), -8, 7) + 8; 18 bytes = d (little endian) then 16
 *     bytes whose byte j holds q_j (low nibble) and q_{j+16} (high nibble).
 *   - 8-bit activations: per 32-block d = amax/127 (fp32), q = roundf(x/d).
 *   - Q8_0 weight block (the 8-bit weights of [COMP], decode only): 32
 *     consecutive K-elements; d = fp16(amax/127); q = clamp(roundf(w/d),
 *     -127, 127); 34 bytes = d (little endian) then the 32 int8 codes.
 *   - Experts: SwiGLU FFN  down( silu(gate x) * (up x) ).
 *   - Router: logits = x . W_r (+ bias), top-k by (logit desc, index asc),
 *     weights = softmax over the k selected logits.  Optional always-on
 *     shared expert with weight 1.
 *   - Where a float result decides an integer (top-k selection, int8 codes of
 *     the activations) both the oracle and the GPU evaluate the same fp32
 *     program, defined here: see tree_sum(), router_logit(), exp_p(),
 *     w4a8_row(), rmsnorm_row().
 *   - The prefill's float path has two statements here: the exact layer in
 *     binary64 (orc_prefill_ref), and the library's rounding points of the
 *     grouped GEMM -- weights, h and routed outputs in bf16, the float32
 *     combine in slot order -- with sums in binary64 (orc_prefill_bf16).
 *
 * Every function works on host memory owned by the caller; no allocation
 * survives a call.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BLK 32          /* elements per quantisation block */
#define ORC_Q4_BYTES 18     /* bytes per Q4_0 block            */
#define ORC_Q8W_BYTES 34    /* bytes per Q8_0 weight block     */

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> binary32, written from the format definition.       */
/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;        */
/* subnormals have exponent field 0 and value frac * 2^-24.                  */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Round-to-nearest-even conversion, subnormals kept, overflow -> inf. */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t x = f32_bits(f);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u)                      /* inf or nan */
        return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x0200u : 0u));
    int e = (int)(ax >> 23) - 127;              /* unbiased exponent of f */
    if (e >= -14) {                             /* normal binary16 range (or overflow) */
        uint32_t frac = ax & 0x7fffffu;
        uint32_t v = ((uint32_t)(e + 15) << 10) | (frac >> 13);
        uint32_t rem = frac & 0x1fffu;          /* 13 dropped bits */
        if (rem > 0x1000u || (rem == 0x1000u && (v & 1u)))
            v += 1u;                            /* carry may bump the exponent */
        if (v >= 0x7c00u) v = 0x7c00u;          /* rounds past the largest finite */
        return (uint16_t)(sign | v);
    }
    if (e < -25) return (uint16_t)sign;         /* below half the smallest subnormal */
    /* subnormal result: value / 2^-24 = mant * 2^(e+1), mant has 24 bits */
    uint32_t mant = (ax & 0x7fffffu) | 0x800000u;
    int shift = -(e + 1);                       /* 14 .. 24 */
    uint32_t q = mant >> shift;
    uint32_t rem = mant & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;                                /* may become 0x400 = smallest normal */
    return (uint16_t)(sign | q);
}

float orc_f16_to_f32(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t ex = ((uint32_t)h >> 10) & 0x1fu;
    uint32_t frac = (uint32_t)h & 0x3ffu;
    if (ex == 0x1fu)
        return bits_f32(sign | 0x7f800000u | (frac << 13));
    if (ex != 0)
        return bits_f32(sign | ((ex - 15u + 127u) << 23) | (frac << 13));
    /* zero or subnormal: frac * 2^-24, exact in binary32 */
    float v = ldexpf((float)frac, -24);
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Pairwise tree sum (the one summation shape used by every pinned program). */
/* Pad v[0..n) with +0.0 up to the next power of two m, then repeatedly       */
/* replace v[i] <- v[2i] + v[2i+1] until one value is left.  n = 1 returns    */
/* v[0] untouched.  `buf` must hold m floats; v may alias buf.                */
/* ------------------------------------------------------------------------ */
static size_t next_pow2(size_t n) { size_t m = 1; while (m < n) m <<= 1; return m; }

static float tree_sum(float *buf, size_t n)
{
    size_t m = next_pow2(n);
    for (size_t i = n; i < m; i++) buf[i] = 0.0f;
    while (m > 1) {
        for (size_t i = 0; i < m / 2; i++) buf[i] = buf[2 * i] + buf[2 * i + 1];
        m /= 2;
    }
    return buf[0];
}

float orc_tree_sum(const float *v, int64_t n)
{
    if (n <= 0) return 0.0f;
    size_t m = next_pow2((size_t)n);
    float *buf = (float *)malloc(m * sizeof(float));
    memcpy(buf, v, (size_t)n * sizeof(float));
    float r = tree_sum(buf, (size_t)n);
    free(buf);
    return r;
}

/* ------------------------------------------------------------------------ */
/* Q4_0 weights [FERMI Methodology 2: group-wise symmetric 4-bit, Q4_0].     */
/* ------------------------------------------------------------------------ */

size_t orc_q4_row_bytes(int64_t K) { return (size_t)(K / ORC_BLK) * ORC_Q4_BYTES; }

/* w: [rows][K] fp32 row-major, K % 32 == 0.  out: rows * (K/32) * 18 bytes. */
void orc_q4_pack(const float *w, int64_t rows, int64_t K, uint8_t *out)
{
    int64_t nb = K / ORC_BLK;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *v = w + r * K + b * ORC_BLK;
            float amax = 0.0f;
            for (int j = 0; j < ORC_BLK; j++) {
                float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            float d32 = amax / 7.0f;
            uint16_t dh = orc_f32_to_f16(d32);
            float df = orc_f16_to_f32(dh);
            uint8_t q[ORC_BLK];
            for (int j = 0; j < ORC_BLK; j++) {
                if (df == 0.0f) { q[j] = 8; continue; }
                float t = roundf(v[j] / df);          /* half away from zero */
                if (t < -8.0f) t = -8.0f;
                if (t > 7.0f) t = 7.0f;
                q[j] = (uint8_t)((int)t + 8);
            }
            uint8_t *blk = out + (r * nb + b) * ORC_Q4_BYTES;
            blk[0] = (uint8_t)(dh & 0xffu);
            blk[1] = (uint8_t)(dh >> 8);
            for (int j = 0; j < 16; j++)
                blk[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
        }
    }
}

/* Unsigned code q (0..15) of element j of one block. */
static int q4_code(const uint8_t *blk, int j)
{
    uint8_t byte = blk[2 + (j & 15)];
    return (j < 16) ? (byte & 0x0f) : (byte >> 4);
}

static float q4_scale(const uint8_t *blk)
{
    return orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
}

/* Dequantised value (q-8)*d.  A 4-bit integer times an 11-bit significand:
 * exact in binary32 and binary64. */
void orc_q4_dequant(const uint8_t *packed, int64_t rows, int64_t K, float *out)
{
    int64_t nb = K / ORC_BLK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = packed + (r * nb + b) * ORC_Q4_BYTES;
            float d = q4_scale(blk);
            for (int j = 0; j < ORC_BLK; j++)
                out[r * K + b * ORC_BLK + j] = (float)(q4_code(blk, j) - 8) * d;
        }
}

/* ------------------------------------------------------------------------ */
/* Q8_0 weights [COMP abstract: 8-bit weights, against which 4-bit decode    */
/* was measured slower on Fermi].  The page names 8-bit weights but no       */
/* format; the plain reading, by analogy with Q4_0: per 32 elements          */
/* d = fp16(amax/127), q = clamp(roundf(w/d), -127, 127), weight = q*d.      */
/* The clamp only acts when d is an fp16 subnormal (relative rounding of d   */
/* up to 1/2 ulp of 2^-24); for normal d, |w/d| <= 127*(1 + 2^-11) < 127.5.  */
/* ------------------------------------------------------------------------ */

size_t orc_q8w_row_bytes(int64_t K) { return (size_t)(K / ORC_BLK) * ORC_Q8W_BYTES; }

/* w: [rows][K] fp32 row-major, K % 32 == 0.  out: rows * (K/32) * 34 bytes. */
void orc_q8w_pack(const float *w, int64_t rows, int64_t K, uint8_t *out)
{
    int64_t nb = K / ORC_BLK;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *v = w + r * K + b * ORC_BLK;
            float amax = 0.0f;
            for (int j = 0; j < ORC_BLK; j++) {
                float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            float d32 = amax / 127.0f;
            uint16_t dh = orc_f32_to_f16(d32);
            float df = orc_f16_to_f32(dh);
            uint8_t *blk = out + (r * nb + b) * ORC_Q8W_BYTES;
            blk[0] = (uint8_t)(dh & 0xffu);
            blk[1] = (uint8_t)(dh >> 8);
            for (int j = 0; j < ORC_BLK; j++) {
                float t = (df == 0.0f) ? 0.0f : roundf(v[j] / df);   /* half away from zero */
                if (t < -127.0f) t = -127.0f;
                if (t > 127.0f) t = 127.0f;
                blk[2 + j] = (uint8_t)(int8_t)(int)t;
            }
        }
    }
}

static int q8w_code(const uint8_t *blk, int j) { return (int)(int8_t)blk[2 + j]; }

static float q8w_scale(const uint8_t *blk)
{
    return orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
}

/* Dequantised value q*d: an 8-bit integer times an 11-bit significand, exact
 * in binary32 and binary64. */
void orc_q8w_dequant(const uint8_t *packed, int64_t rows, int64_t K, float *out)
{
    int64_t nb = K / ORC_BLK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = packed + (r * nb + b) * ORC_Q8W_BYTES;
            float d = q8w_scale(blk);
            for (int j = 0; j < ORC_BLK; j++)
                out[r * K + b * ORC_BLK + j] = (float)q8w_code(blk, j) * d;
        }
}

/* ------------------------------------------------------------------------ */
/* 8-bit activations [FERMI Methodology 1-2: W4A8, 8-bit activations].       */
/* ------------------------------------------------------------------------ */

/* x: [rows][K]; q: [rows][K] int8; d: [rows][K/32] fp32. */
void orc_q8_quantize(const float *x, int64_t rows, int64_t K, int8_t *q, float *d)
{
    int64_t nb = K / ORC_BLK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            const float *v = x + r * K + b * ORC_BLK;
            float amax = 0.0f;
            for (int j = 0; j < ORC_BLK; j++) {
                float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            float dd = amax / 127.0f;
            d[r * nb + b] = dd;
            for (int j = 0; j < ORC_BLK; j++)
                q[r * K + b * ORC_BLK + j] =
                    (dd == 0.0f) ? (int8_t)0 : (int8_t)roundf(v[j] / dd);
        }
}

/* ------------------------------------------------------------------------ */
/* exp_p: the fp32 exponential both sides evaluate (it feeds int8 codes).    */
/* Method: Cody & Waite additive range reduction (W. J. Cody, W. Waite,      */
/* "Software Manual for the Elementary Functions", 1980):                    */
/*   n = rint(x * log2(e)),  r = x - n*ln2  (ln2 split in a hi part with 15  */
/*   significant bits, so n*hi is exact for |n| < 2^9, plus a lo part),      */
/*   exp(x) = 2^n * exp(r),  |r| <= ln2/2,                                   */
/* and exp(r) by its Taylor polynomial of degree 7 (coefficients 1/i!        */
/* rounded to fp32) evaluated by Horner's rule with fused multiply-adds.     */
/* Inputs are clamped to [-104, 89]: exp(-104) is below half the smallest    */
/* fp32 subnormal and exp(89) is above FLT_MAX, so ldexpf gives 0 and +inf.  */
/* ------------------------------------------------------------------------ */
#define EXPP_LOG2E 1.44269502162933349609375f        /* fp32(1/ln 2)          */
#define EXPP_LN2_HI 0.693145751953125f               /* ln 2 to 15 bits      */
#define EXPP_LN2_LO 1.428606765330187045e-06f        /* fp32(ln 2 - LN2_HI)  */

float orc_exp_p(float x)
{
    static const float c[8] = {
        1.0f, 1.0f, 0.5f, (float)(1.0 / 6.0), (float)(1.0 / 24.0),
        (float)(1.0 / 120.0), (float)(1.0 / 720.0), (float)(1.0 / 5040.0)};
    x = fminf(fmaxf(x, -104.0f), 89.0f);
    float n = rintf(x * EXPP_LOG2E);
    float r = fmaf(-n, EXPP_LN2_HI, x);
    r = fmaf(-n, EXPP_LN2_LO, r);
    float p = c[7];
    for (int i = 6; i >= 0; i--) p = fmaf(p, r, c[i]);
    return ldexpf(p, (int)n);
}

/* silu(g) = g * sigmoid(g), evaluated as g / (1 + exp_p(-g)). */
float orc_silu_p(float g) { return g / (1.0f + orc_exp_p(-g)); }

/* ------------------------------------------------------------------------ */
/* Router [FERMI Methodology 1: the prefill GEMM is the MoE's routed grouped  */
/* GEMM; routing itself is the library's definition, see file header].       */
/* ------------------------------------------------------------------------ */

/* logit(t,e): for each 32-wide chunk c of the hidden dimension, a sequential
 * fused multiply-add chain starting from +0.0 over i = 0..31; the chunk
 * partials are then summed by tree_sum(); the bias (if any) is added last. */
static float router_logit(const float *xt, const float *Wr, int64_t H, int64_t E,
                          int64_t e, const float *bias, float *buf)
{
    int64_t nc = H / ORC_BLK;
    for (int64_t c = 0; c < nc; c++) {
        float acc = 0.0f;
        for (int i = 0; i < ORC_BLK; i++) {
            int64_t h = c * ORC_BLK + i;
            acc = fmaf(xt[h], Wr[h * E + e], acc);
        }
        buf[c] = acc;
    }
    float l = tree_sum(buf, (size_t)nc);
    if (bias) l = l + bias[e];
    return l;
}

/* x: [T][H] fp32 (bf16 inputs are widened exactly by the caller);
 * Wr: [H][E] fp32 row-major; bias: [E] or NULL; logits: [T][E]. */
void orc_router_logits(const float *x, int64_t T, int64_t H, const float *Wr,
                       int64_t E, const float *bias, float *logits)
{
    float *buf = (float *)malloc(next_pow2((size_t)(H / ORC_BLK)) * sizeof(float));
    for (int64_t t = 0; t < T; t++)
        for (int64_t e = 0; e < E; e++)
            logits[t * E + e] = router_logit(x + t * H, Wr, H, E, e, bias, buf);
    free(buf);
}

/* Top-k and routing weights.  Selection: repeatedly take the largest logit
 * not yet taken; on equal logits the lower expert index wins (strict '>').
 * Slot s holds the s-th pick, so slots run by descending logit.
 * w32: the fp32 program  m = l_0;  e_s = exp_p(l_s - m);
 *      S = ((e_0 + e_1) + e_2) + ...;  w_s = e_s / S.
 * w64: softmax over the k selected logits in binary64 (libm exp).
 * Either output pointer may be NULL. */
void orc_topk(const float *logits, int64_t T, int64_t E, int32_t k,
              int32_t *ids, float *w32, double *w64)
{
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        int32_t *id = ids + t * k;
        for (int32_t s = 0; s < k; s++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            id[s] = (int32_t)best;
            taken[best] = 1;
        }
        if (w32) {
            float m = l[id[0]];
            float ev[1024];
            float S = 0.0f;
            for (int32_t s = 0; s < k; s++) {
                ev[s] = orc_exp_p(l[id[s]] - m);
                S = (s == 0) ? ev[0] : S + ev[s];
            }
            for (int32_t s = 0; s < k; s++) w32[t * k + s] = ev[s] / S;
        }
        if (w64) {
            double m = (double)l[id[0]], S = 0.0;
            for (int32_t s = 0; s < k; s++) S += exp((double)l[id[s]] - m);
            for (int32_t s = 0; s < k; s++)
                w64[t * k + s] = exp((double)l[id[s]] - m) / S;
        }
    }
    free(taken);
}

/* Expert segments: counts[e], offsets[0..E] (exclusive scan), and a stable
 * counting sort of the flat assignments f = t*k + s by expert, visiting f in
 * increasing order, so each segment lists its tokens in increasing order.
 * perm[offsets[e] + r] = f ;  inv_perm[f] = offsets[e] + r. */
void orc_route_permutation(const int32_t *ids, int64_t T, int32_t k, int64_t E,
                           int32_t *counts, int32_t *offsets, int32_t *perm,
                           int32_t *inv_perm)
{
    int64_t n = T * k;
    for (int64_t e = 0; e < E; e++) counts[e] = 0;
    for (int64_t f = 0; f < n; f++) counts[ids[f]]++;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    for (int64_t e = 0; e < E; e++) fill[e] = offsets[e];
    for (int64_t f = 0; f < n; f++) {
        int32_t e = ids[f];
        perm[fill[e]] = (int32_t)f;
        inv_perm[f] = fill[e];
        fill[e]++;
    }
    free(fill);
}

/* ------------------------------------------------------------------------ */
/* Layer description shared by the two forms.                                */
/* Per expert e: gate [I][H/32 blocks], up [I][H/32], down [H][I/32]; experts */
/* stored one after another.  The shared expert (if any) has the same layout. */
/* ------------------------------------------------------------------------ */
typedef struct {
    int64_t H, I, E;
    int32_t k, has_shared;
    const float *w_router;          /* [H][E] */
    const float *bias;              /* [E] or NULL */
    const uint8_t *gate, *up, *down;
    const uint8_t *s_gate, *s_up, *s_down;
    int32_t wfmt;                   /* 0: Q4_0 (every path); 1: Q8_0 (decode only) */
} orc_layer;

static size_t layer_row_bytes(const orc_layer *L, int64_t K)
{
    return L->wfmt ? orc_q8w_row_bytes(K) : orc_q4_row_bytes(K);
}

static const uint8_t *expert_mat(const uint8_t *base, int64_t e, int64_t rows, int64_t K)
{
    return base + (size_t)e * (size_t)rows * orc_q4_row_bytes(K);
}

static const uint8_t *layer_expert_mat(const orc_layer *L, const uint8_t *base, int64_t e,
                                       int64_t rows, int64_t K)
{
    return base + (size_t)e * (size_t)rows * layer_row_bytes(L, K);
}

/* binary64 dot of one dequantised Q4 row with a binary64 vector. */
static double q4_row_dot_f64(const uint8_t *row, int64_t K, const double *v)
{
    double acc = 0.0;
    for (int64_t b = 0; b < K / ORC_BLK; b++) {
        const uint8_t *blk = row + b * ORC_Q4_BYTES;
        double d = (double)q4_scale(blk);
        for (int j = 0; j < ORC_BLK; j++)
            acc += (double)(q4_code(blk, j) - 8) * d * v[b * ORC_BLK + j];
    }
    return acc;
}

/* One SwiGLU expert in binary64:  o = down( silu(gate x) * (up x) ). */
static void expert_ffn_f64(const uint8_t *g, const uint8_t *u, const uint8_t *dn,
                           int64_t H, int64_t I, const double *x, double *hbuf,
                           double *o)
{
    size_t rg = orc_q4_row_bytes(H), rd = orc_q4_row_bytes(I);
    for (int64_t i = 0; i < I; i++) {
        double gi = q4_row_dot_f64(g + i * rg, H, x);
        double ui = q4_row_dot_f64(u + i * rg, H, x);
        hbuf[i] = gi / (1.0 + exp(-gi)) * ui;
    }
    for (int64_t r = 0; r < H; r++) o[r] = q4_row_dot_f64(dn + r * rd, I, hbuf);
}

/* Prefill reference (binary64).  For each listed token t:
 *   y_t = sum_s w64[t,s] * FFN_{ids[t,s]}(x_t)  +  FFN_shared(x_t)
 * with exactly dequantised weights.  x: [T][H] (the bf16 inputs widened);
 * ids/w64 come from the oracle's own routing; tokens: indices into x (NULL
 * means 0..n_tok-1); y: [n_tok][H]. */
void orc_prefill_ref(const orc_layer *L, const float *x, const int32_t *ids,
                     const double *w64, const int64_t *tokens, int64_t n_tok,
                     double *y)
{
    int64_t H = L->H, I = L->I;
    double *xd = (double *)malloc((size_t)H * sizeof(double));
    double *hb = (double *)malloc((size_t)I * sizeof(double));
    double *o = (double *)malloc((size_t)H * sizeof(double));
    for (int64_t n = 0; n < n_tok; n++) {
        int64_t t = tokens ? tokens[n] : n;
        double *yt = y + n * H;
        for (int64_t h = 0; h < H; h++) { xd[h] = (double)x[t * H + h]; yt[h] = 0.0; }
        for (int32_t s = 0; s < L->k; s++) {
            int64_t e = ids[t * L->k + s];
            expert_ffn_f64(expert_mat(L->gate, e, I, H), expert_mat(L->up, e, I, H),
                           expert_mat(L->down, e, H, I), H, I, xd, hb, o);
            for (int64_t h = 0; h < H; h++) yt[h] += w64[t * L->k + s] * o[h];
        }
        if (L->has_shared) {
            expert_ffn_f64(L->s_gate, L->s_up, L->s_down, H, I, xd, hb, o);
            for (int64_t h = 0; h < H; h++) yt[h] += o[h];
        }
    }
    free(xd); free(hb); free(o);
}

/* ------------------------------------------------------------------------ */
/* The bf16 prefill program [FERMI Methodology 1: grouped 4-bit GEMM]         */
/* ------------------------------------------------------------------------ */

/* binary32 -> nearest bfloat16 (the top 16 bits of a binary32; ties to even),
 * returned widened back to binary32.  Infinities, zeros and subnormals follow
 * the same bit rule; a NaN stays a (quiet) NaN. */
float orc_bf16_round(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return bits_f32((u | 0x00400000u) & 0xffff0000u);
    uint32_t base = u & 0xffff0000u, rem = u & 0x0000ffffu;
    if (rem > 0x8000u || (rem == 0x8000u && (base & 0x00010000u)))
        base += 0x00010000u;               /* a carry into the exponent is the next binade */
    return bits_f32(base);
}

void orc_bf16_round_n(const float *x, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_round(x[i]);
}

/* binary64 dot of one Q4 row, each weight (q - 8) * d (exact in binary32)
 * rounded once to bf16, with a binary64 vector. */
static double q4_row_dot_bf16w(const uint8_t *row, int64_t K, const double *v)
{
    double acc = 0.0;
    for (int64_t b = 0; b < K / ORC_BLK; b++) {
        const uint8_t *blk = row + b * ORC_Q4_BYTES;
        float d = q4_scale(blk);
        for (int j = 0; j < ORC_BLK; j++) {
            float w = orc_bf16_round((float)(q4_code(blk, j) - 8) * d);
            acc += (double)w * v[b * ORC_BLK + j];
        }
    }
    return acc;
}

/* One SwiGLU expert of the bf16 program: gate and up over bf16 weights,
 * h = bf16(silu(g) * u), o = down over bf16 weights and h, rounded to
 * binary32 and, for a routed expert (round_o), on to bf16. */
static void expert_ffn_bf16(const uint8_t *g, const uint8_t *u, const uint8_t *dn,
                            int64_t H, int64_t I, const double *x, double *hbuf,
                            float *o, int round_o)
{
    size_t rg = orc_q4_row_bytes(H), rd = orc_q4_row_bytes(I);
    for (int64_t i = 0; i < I; i++) {
        double gi = q4_row_dot_bf16w(g + i * rg, H, x);
        double ui = q4_row_dot_bf16w(u + i * rg, H, x);
        hbuf[i] = (double)orc_bf16_round((float)(gi / (1.0 + exp(-gi)) * ui));
    }
    for (int64_t r = 0; r < H; r++) {
        float v = (float)q4_row_dot_bf16w(dn + r * rd, I, hbuf);
        o[r] = round_o ? orc_bf16_round(v) : v;
    }
}

/* The library's bf16 prefill program (the rounding points of the grouped
 * GEMM; the pages give the GEMM and no precision).  For each listed token t,
 * x_t already bf16 (widened): every weight is (q - 8) * d rounded once to
 * bf16; gate, up and down sums are exact-ish (binary64 here, any order on
 * the GPU); h = bf16(silu(g) * u); a routed expert's output is rounded to
 * bf16, the shared expert's to binary32; then, in binary32 and in this order,
 *   y_t = (((o_shared + w[t,0] * o_0) + w[t,1] * o_1) + ...)
 * with w the binary32 routing weights (o_shared = 0 without a shared expert).
 * x: [T][H]; ids, w32: [T][k]; tokens: indices into x (NULL: 0..n_tok-1);
 * y: [n_tok][H] binary32. */
void orc_prefill_bf16(const orc_layer *L, const float *x, const int32_t *ids,
                      const float *w32, const int64_t *tokens, int64_t n_tok,
                      float *y)
{
    int64_t H = L->H, I = L->I;
    double *xd = (double *)malloc((size_t)H * sizeof(double));
    double *hb = (double *)malloc((size_t)I * sizeof(double));
    float *o = (float *)malloc((size_t)H * sizeof(float));
    for (int64_t n = 0; n < n_tok; n++) {
        int64_t t = tokens ? tokens[n] : n;
        float *yt = y + n * H;
        for (int64_t h = 0; h < H; h++) xd[h] = (double)x[t * H + h];
        if (L->has_shared) {
            expert_ffn_bf16(L->s_gate, L->s_up, L->s_down, H, I, xd, hb, o, 0);
            for (int64_t h = 0; h < H; h++) yt[h] = o[h];
        } else {
            for (int64_t h = 0; h < H; h++) yt[h] = 0.0f;
        }
        for (int32_t s = 0; s < L->k; s++) {
            int64_t e = ids[t * L->k + s];
            float ws = w32[t * L->k + s];
            expert_ffn_bf16(expert_mat(L->gate, e, I, H), expert_mat(L->up, e, I, H),
                            expert_mat(L->down, e, H, I), H, I, xd, hb, o, 1);
            for (int64_t h = 0; h < H; h++) {
                float p = ws * o[h];
                yt[h] = yt[h] + p;
            }
        }
    }
    free(xd); free(hb); free(o);
}

/* ------------------------------------------------------------------------ */
/* W4A8 decode [FERMI Methodology 1: W4A8 integer kernel; Key Contribution 2] */
/* ------------------------------------------------------------------------ */

/* One Q4 row against int8 activations.  Block b:
 *   dot_b = sum_j (q_w[j] - 8) * q_a[j]        exact integer, |dot_b| <= 32512
 *   p_b   = (d_w[b] * d_a[b]) * (float)dot_b   two fp32 multiplies
 * row value = tree_sum(p_0 .. p_{nb-1}).  `dots` (nb entries) may be NULL. */
static float w4a8_row(const uint8_t *row, int64_t K, const int8_t *qa,
                      const float *da, int32_t *dots, float *buf)
{
    int64_t nb = K / ORC_BLK;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *blk = row + b * ORC_Q4_BYTES;
        int32_t dot = 0;
        for (int j = 0; j < ORC_BLK; j++)
            dot += (int32_t)(q4_code(blk, j) - 8) * (int32_t)qa[b * ORC_BLK + j];
        if (dots) dots[b] = dot;
        float s = q4_scale(blk) * da[b];
        buf[b] = s * (float)dot;
    }
    return tree_sum(buf, (size_t)nb);
}

/* One Q8_0 row against int8 activations (W8A8): the W4A8 program with the
 * signed codes in place of q - 8.  Block b:
 *   dot_b = sum_j q_w[j] * q_a[j]               exact integer, |dot_b| <= 516128
 *   p_b   = (d_w[b] * d_a[b]) * (float)dot_b    two fp32 multiplies
 * row value = tree_sum(p_0 .. p_{nb-1}). */
static float w8a8_row(const uint8_t *row, int64_t K, const int8_t *qa,
                      const float *da, int32_t *dots, float *buf)
{
    int64_t nb = K / ORC_BLK;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *blk = row + b * ORC_Q8W_BYTES;
        int32_t dot = 0;
        for (int j = 0; j < ORC_BLK; j++)
            dot += (int32_t)q8w_code(blk, j) * (int32_t)qa[b * ORC_BLK + j];
        if (dots) dots[b] = dot;
        float s = q8w_scale(blk) * da[b];
        buf[b] = s * (float)dot;
    }
    return tree_sum(buf, (size_t)nb);
}

/* W: [N] Q8_0 rows of K/32 blocks; as orc_w4a8_gemv. */
void orc_w8a8_gemv(const uint8_t *W, int64_t N, int64_t K, const int8_t *qa,
                   const float *da, int32_t *dots, float *out)
{
    int64_t nb = K / ORC_BLK;
    float *buf = (float *)malloc(next_pow2((size_t)nb) * sizeof(float));
    for (int64_t r = 0; r < N; r++)
        out[r] = w8a8_row(W + r * orc_q8w_row_bytes(K), K, qa, da,
                          dots ? dots + r * nb : NULL, buf);
    free(buf);
}

/* The decode row program of the layer's weight format. */
static float layer_row(const orc_layer *L, const uint8_t *row, int64_t K, const int8_t *qa,
                       const float *da, float *buf)
{
    return L->wfmt ? w8a8_row(row, K, qa, da, NULL, buf) : w4a8_row(row, K, qa, da, NULL, buf);
}

/* W: [N] rows of K/32 blocks; qa [K], da [K/32]; dots [N][K/32] or NULL;
 * out [N]. */
void orc_w4a8_gemv(const uint8_t *W, int64_t N, int64_t K, const int8_t *qa,
                   const float *da, int32_t *dots, float *out)
{
    int64_t nb = K / ORC_BLK;
    float *buf = (float *)malloc(next_pow2((size_t)nb) * sizeof(float));
    for (int64_t r = 0; r < N; r++)
        out[r] = w4a8_row(W + r * orc_q4_row_bytes(K), K, qa, da,
                          dots ? dots + r * nb : NULL, buf);
    free(buf);
}

/* Optional intermediate values of one decode step (every pointer may be NULL).
 * Slot k is the shared expert when the layer has one. */
typedef struct {
    float *logits;        /* [E]                   */
    int32_t *ids;         /* [k]                   */
    float *w;             /* [k]                   */
    int8_t *qx;           /* [H]                   */
    float *dx;            /* [H/32]                */
    float *gate, *up;     /* [k+S][I]              */
    int8_t *qh;           /* [k+S][I]              */
    float *dh;            /* [k+S][I/32]           */
    float *o;             /* [k+S][H]              */
} orc_decode_trace;

/* One decode step (fp32 program, the target of bit-exact comparison); with
 * Q8_0 weights (wfmt = 1) every row program below is w8a8_row:
 *   logits, ids, w      router_logit + orc_topk (fp32 weights)
 *   qx, dx = q8(x)
 *   per slot expert (and the shared one):
 *     g_i, u_i = w4a8_row(gate_i | up_i, qx, dx)
 *     h_i = silu_p(g_i) * u_i ;  qh, dh = q8(h)
 *     o_r = w4a8_row(down_r, qh, dh)
 *   y_r = ((w_0*o_0r + w_1*o_1r) + ... + w_{k-1}*o_{k-1,r}) + o_shared_r
 *   (each product rounded, sums left to right). */
void orc_decode(const orc_layer *L, const float *x, float *y, orc_decode_trace *tr)
{
    int64_t H = L->H, I = L->I, E = L->E;
    int32_t k = L->k, S = L->has_shared ? 1 : 0;
    float *logits = (float *)malloc((size_t)E * sizeof(float));
    int32_t ids[1024];
    float w[1024];
    int8_t *qx = (int8_t *)malloc((size_t)H);
    float *dx = (float *)malloc((size_t)(H / ORC_BLK) * sizeof(float));
    float *g = (float *)malloc((size_t)I * sizeof(float));
    float *u = (float *)malloc((size_t)I * sizeof(float));
    float *h = (float *)malloc((size_t)I * sizeof(float));
    int8_t *qh = (int8_t *)malloc((size_t)I);
    float *dh = (float *)malloc((size_t)(I / ORC_BLK) * sizeof(float));
    float *o = (float *)malloc((size_t)(k + S) * (size_t)H * sizeof(float));
    size_t nbmax = next_pow2((size_t)((H > I ? H : I) / ORC_BLK));
    float *buf = (float *)malloc(nbmax * sizeof(float));

    orc_router_logits(x, 1, H, L->w_router, E, L->bias, logits);
    orc_topk(logits, 1, E, k, ids, w, NULL);
    orc_q8_quantize(x, 1, H, qx, dx);
    for (int32_t s = 0; s < k + S; s++) {
        const uint8_t *G, *U, *D;
        if (s < k) {
            G = layer_expert_mat(L, L->gate, ids[s], I, H);
            U = layer_expert_mat(L, L->up, ids[s], I, H);
            D = layer_expert_mat(L, L->down, ids[s], H, I);
        } else {
            G = L->s_gate; U = L->s_up; D = L->s_down;
        }
        for (int64_t i = 0; i < I; i++) {
            g[i] = layer_row(L, G + i * layer_row_bytes(L, H), H, qx, dx, buf);
            u[i] = layer_row(L, U + i * layer_row_bytes(L, H), H, qx, dx, buf);
            h[i] = orc_silu_p(g[i]) * u[i];
        }
        orc_q8_quantize(h, 1, I, qh, dh);
        for (int64_t r = 0; r < H; r++)
            o[s * H + r] = layer_row(L, D + r * layer_row_bytes(L, I), I, qh, dh, buf);
        if (tr) {
            if (tr->gate) memcpy(tr->gate + s * I, g, (size_t)I * sizeof(float));
            if (tr->up) memcpy(tr->up + s * I, u, (size_t)I * sizeof(float));
            if (tr->qh) memcpy(tr->qh + s * I, qh, (size_t)I);
            if (tr->dh) memcpy(tr->dh + s * (I / ORC_BLK), dh,
                               (size_t)(I / ORC_BLK) * sizeof(float));
        }
    }
    for (int64_t r = 0; r < H; r++) {
        float acc = w[0] * o[r];
        for (int32_t s = 1; s < k; s++) acc = acc + w[s] * o[s * H + r];
        if (S) acc = acc + o[k * H + r];
        y[r] = acc;
    }
    if (tr) {
        if (tr->logits) memcpy(tr->logits, logits, (size_t)E * sizeof(float));
        if (tr->ids) memcpy(tr->ids, ids, (size_t)k * sizeof(int32_t));
        if (tr->w) memcpy(tr->w, w, (size_t)k * sizeof(float));
        if (tr->qx) memcpy(tr->qx, qx, (size_t)H);
        if (tr->dx) memcpy(tr->dx, dx, (size_t)(H / ORC_BLK) * sizeof(float));
        if (tr->o) memcpy(tr->o, o, (size_t)(k + S) * (size_t)H * sizeof(float));
    }
    free(logits); free(qx); free(dx); free(g); free(u); free(h);
    free(qh); free(dh); free(o); free(buf);
}

/* ------------------------------------------------------------------------ */
/* RMSNorm between stacked layers (unit gain):  out = y / sqrt(mean(y^2)+eps) */
/* Sum of squares: per 32-chunk sequential fmaf(y, y, acc) from +0.0, chunk   */
/* partials by tree_sum(); mean = ss / H; r = sqrtf(mean + eps); out = y / r. */
/* ------------------------------------------------------------------------ */
void orc_rmsnorm(const float *y, int64_t T, int64_t H, float eps, float *out)
{
    int64_t nc = H / ORC_BLK;
    float *buf = (float *)malloc(next_pow2((size_t)nc) * sizeof(float));
    for (int64_t t = 0; t < T; t++) {
        const float *v = y + t * H;
        for (int64_t c = 0; c < nc; c++) {
            float acc = 0.0f;
            for (int i = 0; i < ORC_BLK; i++)
                acc = fmaf(v[c * ORC_BLK + i], v[c * ORC_BLK + i], acc);
            buf[c] = acc;
        }
        float ss = tree_sum(buf, (size_t)nc);
        float r = sqrtf(ss / (float)H + eps);
        for (int64_t h = 0; h < H; h++) out[t * H + h] = v[h] / r;
    }
    free(buf);
}
