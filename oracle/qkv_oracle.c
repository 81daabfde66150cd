/*
 * qkv_oracle.c -- CPU oracle of the attention-input epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes is the UNFUSED chain the fused kernel replaces, as the page
 * "73 · D3-8 — G4 FusedQKV ported to CUDA" (minfer CUDA optimization steps)
 * describes it in §2 ("The fusion's bitwise legitimacy") and §3.2 Excerpt A:
 *
 *   add_bias on q, then k, then v        (one f32 add per element)
 *   rope on q, then rope on k            (NeoX pairing: element i with i+half)
 *   store K, then store V into the cache (row = position, dst[pos*nkt + j])
 *
 * and the q/k-norm variant (per-head RMS norm of q and k between the bias add
 * and the rope, see oracle_rms_norm_heads).  The rope style (0 = NeoX,
 * 1 = interleaved pairs (2i, 2i+1)) and a frequency scale are parameters of
 * both chains.
 *
 * Each step is its own plain loop, in that order, written for a reader to check
 * against the page by eye.  The per-pair cos/sin are recomputed inside the rope
 * loop exactly as the unfused rope kernel does (nothing is hoisted or blocked).
 *
 * Readings taken where the pages leave a step open:
 *   - inverse frequency inv[i] = theta^(-2i/hd) is the correctly rounded f32
 *     of that real number: computed with libm pow in double, rounded once;
 *   - angle a = f32(pos * inv[i]): one f32 multiply, as the page's kernel does;
 *   - c = f32(cos(double a)), s = f32(sin(double a)): double libm, rounded once;
 *   - each rotated output is f32((double)x0*c -/+ (double)x1*s): the products
 *     are exact in double, the sum is rounded once in double, then to f32;
 *   - the f16 cache store is IEEE binary16 round-to-nearest-even with
 *     subnormals kept and overflow to infinity (the page says __float2half,
 *     which is round-to-nearest);
 *   - the k section is roped with the q formula and BOTH halves are written
 *     back and stored (the page elides the k branch body);
 *   - a token's cache row is slot*n_ctx + pos (slot 0 when no slot array is
 *     given); a position outside [0, n_ctx) or a slot outside [0, n_slots) is
 *     an error and writes no row ("07 · The allocator", §3.2 Excerpt 8 and the
 *     invariants list of §3.4: a position >= n_ctx is a hard error).
 *
 * Build with -O2 -ffp-contract=off and no fast-math so every operation rounds
 * as written.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------------------
 * Step O1 -- add_bias: x[t][j] = f32(x[t][j] + b[j]) for j < width.
 * Page 73 §3.2 Excerpt A: "q[j] + bias_q[j]", "v[j] + bias_v[j]"; §2 calls it
 * the same two-operand one-add as the unfused add_bias kernel.
 * ------------------------------------------------------------------------- */
void oracle_add_bias(float *x, const float *b, int64_t nt, int64_t width,
                     int64_t ld)
{
    for (int64_t t = 0; t < nt; ++t)
        for (int64_t j = 0; j < width; ++j)
            x[t * ld + j] = x[t * ld + j] + b[j];
}

/* ---------------------------------------------------------------------------
 * Step O2 -- inverse frequencies: inv[i] = theta^(-2i/hd), i < hd/2.
 * Page 73 §3.2 Excerpt A forms freq = freq_scale / powf(freq_base, 2d/hd) with
 * freq_scale = 1 here; the value taken is the correctly rounded f32 of the
 * real number theta^(-2i/hd).
 * ------------------------------------------------------------------------- */
void oracle_inv_freq(float theta, int head_dim, float *inv)
{
    int half = head_dim / 2;
    for (int i = 0; i < half; ++i) {
        double e = -(2.0 * (double)i) / (double)head_dim;
        inv[i] = (float)pow((double)theta, e);
    }
}

/* Step O2 with a frequency scale (the page's kernel multiplies by
 * freq_scale, §3.2 Excerpt A): inv[i] = f32(freq_scale * theta^(-2i/hd)),
 * the product taken in double and rounded once. */
void oracle_inv_freq_scaled(float theta, float freq_scale, int head_dim, float *inv)
{
    int half = head_dim / 2;
    for (int i = 0; i < half; ++i) {
        double e = -(2.0 * (double)i) / (double)head_dim;
        inv[i] = (float)((double)freq_scale * pow((double)theta, e));
    }
}

/* ---------------------------------------------------------------------------
 * Step O3 -- rope, NeoX pairing, on one section holding n_heads heads of
 * head_dim elements per token row (row stride ld elements).
 * Page 73 §3.2 Excerpt A: j = head*hd + d, j2 = j + hd/2, angle pos*freq,
 * out[j] = x0*cos - x1*sin, out[j2] = x0*sin + x1*cos, in place.
 * ------------------------------------------------------------------------- */
void oracle_rope_neox(float *x, int64_t nt, int64_t ld, int n_heads,
                      int head_dim, const int32_t *pos, const float *inv)
{
    int half = head_dim / 2;
    for (int64_t t = 0; t < nt; ++t) {
        for (int h = 0; h < n_heads; ++h) {
            float *row = x + t * ld + (int64_t)h * head_dim;
            for (int i = 0; i < half; ++i) {
                float a = (float)pos[t] * inv[i];
                float c = (float)cos((double)a);
                float s = (float)sin((double)a);
                float x0 = row[i];
                float x1 = row[i + half];
                row[i]        = (float)((double)x0 * c - (double)x1 * s);
                row[i + half] = (float)((double)x0 * s + (double)x1 * c);
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Step O3' -- rope with interleaved (GPT-J) pairing: inside each head, pair i
 * is (x[2i], x[2i+1]) and turns by pos*inv[i].  Page "06 · Assign + fusion"
 * §3.2 names the style (RopeStyle other than NonInterleaved); the rotation is
 * the NeoX one applied to adjacent elements.
 * ------------------------------------------------------------------------- */
void oracle_rope_interleaved(float *x, int64_t nt, int64_t ld, int n_heads,
                             int head_dim, const int32_t *pos, const float *inv)
{
    int half = head_dim / 2;
    for (int64_t t = 0; t < nt; ++t) {
        for (int h = 0; h < n_heads; ++h) {
            float *row = x + t * ld + (int64_t)h * head_dim;
            for (int i = 0; i < half; ++i) {
                float a = (float)pos[t] * inv[i];
                float c = (float)cos((double)a);
                float s = (float)sin((double)a);
                float x0 = row[2 * i];
                float x1 = row[2 * i + 1];
                row[2 * i]     = (float)((double)x0 * c - (double)x1 * s);
                row[2 * i + 1] = (float)((double)x0 * s + (double)x1 * c);
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Step P -- the concat QKV projection that feeds the epilogue.  The page
 * "73 · D3-8" §2 ("Why the concat matmul is bitwise") and Excerpt C describe
 * one matmul over the concat weight rows wq|wk|wv producing the q|k|v row of
 * each token.  Here the activations and weights are bfloat16 (raw bits) and
 *   y[t][n] = f32( sum_k x[t][k] * w[n][k] ),
 * the products exact in double, the sum taken in double in k order, rounded
 * once to f32.  w is [n_out][hidden] (one row per output feature); y is
 * [nt][n_out] with row stride ld_y.
 * ------------------------------------------------------------------------- */
static double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void oracle_proj_bf16(const uint16_t *x, int64_t ld_x, const uint16_t *w,
                      int64_t nt, int64_t n_out, int64_t hidden,
                      float *y, int64_t ld_y)
{
    for (int64_t t = 0; t < nt; ++t) {
        for (int64_t n = 0; n < n_out; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < hidden; ++k)
                acc += oracle_bf16_to_double(x[t * ld_x + k]) *
                       oracle_bf16_to_double(w[n * hidden + k]);
            y[t * ld_y + n] = (float)acc;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Step P with 8-bit float weights (weight-only quantisation of the same
 * matmul).  Reading, since the page's own weights are block-quantised and it
 * fixes no 8-bit format: every weight is an OCP 8-bit float in the E4M3
 * encoding -- sign bit, 4 exponent bits with bias 7, 3 mantissa bits; an
 * exponent field of 0 holds the subnormals m * 2^-9; the two patterns with
 * all exponent and mantissa bits set (0x7f, 0xff) are NaN; there is no
 * infinity -- and each weight row n carries one f32 scale s[n]:
 *   y[t][n] = f32( s[n] * sum_k x[t][k] * e4m3(w[n][k]) ),
 * x bfloat16 as above, the products exact in double, the sum in double in k
 * order, times the scale in double, rounded once to f32.
 * ------------------------------------------------------------------------- */
static double oracle_e4m3_to_double(uint8_t b)
{
    const int sign = b >> 7;
    const int e = (b >> 3) & 15;
    const int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);               /* m/8 * 2^(1-7) */
    else
        v = ldexp((double)(8 + m), e - 10);     /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

void oracle_e4m3_decode(const uint8_t *b, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_to_double(b[i]);
}

void oracle_proj_fp8w(const uint16_t *x, int64_t ld_x, const uint8_t *w,
                      const float *scale, int64_t nt, int64_t n_out,
                      int64_t hidden, float *y, int64_t ld_y)
{
    /* the value of each of the 256 codes, decoded once per call (a code's
     * value depends on nothing else) */
    double val[256];
    for (int c = 0; c < 256; ++c)
        val[c] = oracle_e4m3_to_double((uint8_t)c);
    for (int64_t t = 0; t < nt; ++t) {
        for (int64_t n = 0; n < n_out; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < hidden; ++k)
                acc += oracle_bf16_to_double(x[t * ld_x + k]) * val[w[n * hidden + k]];
            y[t * ld_y + n] = (float)((double)scale[n] * acc);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Step N -- per-head RMS norm (the q/k norm of the Qwen3-style variant).
 * Page "06 · Assign + fusion" §3.2 lists a per-head q/k norm op (QkNorm) and
 * the fused FusedQkvNorm, "the Qwen3 per-head-norm variant", without a
 * formula.  Reading: over each head's head_dim values,
 *   y[j] = x[j] / sqrt(mean_j(x[j]^2) + eps) * w[j]
 * with one [head_dim] weight shared by the heads of the section, evaluated in
 * double (the squares of f32 values are exact there) and rounded once to f32.
 * ------------------------------------------------------------------------- */
void oracle_rms_norm_heads(float *x, int64_t nt, int64_t ld, int n_heads,
                           int head_dim, const float *w, float eps)
{
    for (int64_t t = 0; t < nt; ++t) {
        for (int h = 0; h < n_heads; ++h) {
            float *row = x + t * ld + (int64_t)h * head_dim;
            double ss = 0.0;
            for (int j = 0; j < head_dim; ++j)
                ss += (double)row[j] * (double)row[j];
            double r = 1.0 / sqrt(ss / (double)head_dim + (double)eps);
            for (int j = 0; j < head_dim; ++j)
                row[j] = (float)((double)row[j] * r * (double)w[j]);
        }
    }
}

/* ---------------------------------------------------------------------------
 * f32 -> IEEE 754 binary16, round to nearest, ties to even.  Written from the
 * binary16 definition (1 sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits; subnormals are fraction * 2^-24).  NaN stays a quiet NaN.
 * ------------------------------------------------------------------------- */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, sizeof x);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t exp = (x >> 23) & 0xffu;
    uint32_t man = x & 0x7fffffu;

    if (exp == 0xffu) /* infinity or NaN */
        return (uint16_t)(sign | 0x7c00u | (man ? 0x0200u | (man >> 13) : 0u));

    int e16 = (int)exp - 127 + 15; /* binary16 biased exponent */
    if (e16 >= 31)                 /* |f| >= 2^16: beyond the largest finite */
        return (uint16_t)(sign | 0x7c00u);

    if (e16 <= 0) {
        /* binary16 subnormal (or zero): value = m * 2^-24.  f = mf * 2^(exp-150)
         * with the implicit bit, so m = mf / 2^(126-exp), rounded. */
        if (exp < 102) /* |f| < 2^-25: below half the smallest subnormal */
            return (uint16_t)sign;
        uint32_t mf = man | 0x800000u;
        int shift = 126 - (int)exp; /* 14 .. 24 */
        uint32_t m = mf >> shift;
        uint32_t rem = mf & ((1u << shift) - 1u);
        uint32_t halfway = 1u << (shift - 1);
        if (rem > halfway || (rem == halfway && (m & 1u)))
            m += 1u; /* may carry into the smallest normal: still correct */
        return (uint16_t)(sign | m);
    }

    uint32_t h = sign | ((uint32_t)e16 << 10) | (man >> 13);
    uint32_t rem = man & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u)))
        h += 1u; /* a carry out of the fraction bumps the exponent; 65520 -> inf */
    return (uint16_t)h;
}

/* ---------------------------------------------------------------------------
 * Step O4 -- KV store.  For each token, compute its cache row and the row's
 * contents converted to the cache dtype.  Page 73 §3.2 Excerpt A stores to
 * dst[pos*nkt + j] (f32, or __float2half for an f16 cache); "07 · The
 * allocator" §2.5 lays each per-layer region out as n_ctx rows of nkt
 * elements.  This step writes the converted rows to dense [nt][nkt] arrays
 * plus the row index (-1 when the token's position or slot is out of range);
 * oracle_scatter_rows then writes them into a cache.  Returns the number of
 * tokens that were rejected.
 * cache_dtype: 0 = f32, 1 = f16 (raw binary16 bits).
 * ------------------------------------------------------------------------- */
static int64_t oracle_row_of(const int32_t *pos, const int32_t *slot,
                             int64_t t, int64_t n_ctx, int64_t n_slots)
{
    int64_t p = pos[t];
    int64_t s = slot ? (int64_t)slot[t] : 0;
    if (p < 0 || p >= n_ctx)
        return -1;
    if (s < 0 || s >= n_slots)
        return -1;
    return s * n_ctx + p;
}

int64_t oracle_store_rows(const float *x, int64_t nt, int64_t ld, int64_t nkt,
                          const int32_t *pos, const int32_t *slot,
                          int64_t n_ctx, int64_t n_slots, int cache_dtype,
                          int64_t *row_ids, void *rows)
{
    int64_t rejected = 0;
    for (int64_t t = 0; t < nt; ++t) {
        int64_t r = oracle_row_of(pos, slot, t, n_ctx, n_slots);
        row_ids[t] = r;
        if (r < 0) {
            ++rejected;
            continue;
        }
        for (int64_t j = 0; j < nkt; ++j) {
            float val = x[t * ld + j];
            if (cache_dtype == 0)
                ((float *)rows)[t * nkt + j] = val;
            else
                ((uint16_t *)rows)[t * nkt + j] = oracle_f32_to_f16(val);
        }
    }
    return rejected;
}

/* Write converted rows into a dense cache of n_rows rows (rows with id -1 are
 * skipped). elem_bytes is 4 (f32) or 2 (f16). */
void oracle_scatter_rows(void *cache, int64_t n_rows, int64_t nkt,
                         int elem_bytes, int64_t nt, const int64_t *row_ids,
                         const void *rows)
{
    for (int64_t t = 0; t < nt; ++t) {
        int64_t r = row_ids[t];
        if (r < 0 || r >= n_rows)
            continue;
        memcpy((char *)cache + (r * nkt) * elem_bytes,
               (const char *)rows + (t * nkt) * elem_bytes,
               (size_t)(nkt * elem_bytes));
    }
}

/* ---------------------------------------------------------------------------
 * The whole chain, in the unfused order: add_bias x3, inverse frequencies,
 * rope on q, rope on k, store K, store V.  q/k/v are modified in place (the
 * page's kernel writes all three sections back).  krows/vrows receive the
 * [nt][nkt] cache rows in the cache dtype and row_ids the row written for
 * each token.  Returns the number of tokens whose position or slot was out
 * of range (0 on success); such tokens are still biased and roped.
 * ------------------------------------------------------------------------- */
int64_t oracle_qkv_epilogue(float *q, float *k, float *v,
                            int64_t ld_q, int64_t ld_k, int64_t ld_v,
                            const float *bq, const float *bk, const float *bv,
                            const int32_t *pos, const int32_t *slot,
                            int64_t nt, int n_head, int n_kv_head,
                            int head_dim, float theta,
                            int64_t n_ctx, int64_t n_slots, int cache_dtype,
                            int rope_style, float freq_scale,
                            int64_t *row_ids, void *krows, void *vrows)
{
    int64_t nqt = (int64_t)n_head * head_dim;
    int64_t nkt = (int64_t)n_kv_head * head_dim;
    float inv[4096];
    if (head_dim <= 0 || head_dim % 2 != 0 || head_dim / 2 > 4096)
        return -1;

    oracle_add_bias(q, bq, nt, nqt, ld_q);
    oracle_add_bias(k, bk, nt, nkt, ld_k);
    oracle_add_bias(v, bv, nt, nkt, ld_v);

    if (freq_scale == 1.0f)
        oracle_inv_freq(theta, head_dim, inv);
    else
        oracle_inv_freq_scaled(theta, freq_scale, head_dim, inv);
    if (rope_style == 0) {
        oracle_rope_neox(q, nt, ld_q, n_head, head_dim, pos, inv);
        oracle_rope_neox(k, nt, ld_k, n_kv_head, head_dim, pos, inv);
    } else {
        oracle_rope_interleaved(q, nt, ld_q, n_head, head_dim, pos, inv);
        oracle_rope_interleaved(k, nt, ld_k, n_kv_head, head_dim, pos, inv);
    }

    int64_t bad = oracle_store_rows(k, nt, ld_k, nkt, pos, slot, n_ctx,
                                    n_slots, cache_dtype, row_ids, krows);
    oracle_store_rows(v, nt, ld_v, nkt, pos, slot, n_ctx, n_slots,
                      cache_dtype, row_ids, vrows);
    return bad;
}

/* ---------------------------------------------------------------------------
 * The q/k-norm variant of the chain: optional add_bias (NULL bias = none, as
 * in the Qwen3 attention), per-head RMS norm of q (weight wq) and of k (weight
 * wk), then rope on q and k, then store K and V.  v is never normalised.
 * Returns as oracle_qkv_epilogue.
 * ------------------------------------------------------------------------- */
int64_t oracle_qkv_norm_epilogue(float *q, float *k, float *v,
                                 int64_t ld_q, int64_t ld_k, int64_t ld_v,
                                 const float *bq, const float *bk, const float *bv,
                                 const float *wq, const float *wk, float eps,
                                 const int32_t *pos, const int32_t *slot,
                                 int64_t nt, int n_head, int n_kv_head,
                                 int head_dim, float theta,
                                 int64_t n_ctx, int64_t n_slots, int cache_dtype,
                                 int rope_style, float freq_scale,
                                 int64_t *row_ids, void *krows, void *vrows)
{
    int64_t nqt = (int64_t)n_head * head_dim;
    int64_t nkt = (int64_t)n_kv_head * head_dim;
    float inv[4096];
    if (head_dim <= 0 || head_dim % 2 != 0 || head_dim / 2 > 4096)
        return -1;

    if (bq)
        oracle_add_bias(q, bq, nt, nqt, ld_q);
    if (bk)
        oracle_add_bias(k, bk, nt, nkt, ld_k);
    if (bv)
        oracle_add_bias(v, bv, nt, nkt, ld_v);

    oracle_rms_norm_heads(q, nt, ld_q, n_head, head_dim, wq, eps);
    oracle_rms_norm_heads(k, nt, ld_k, n_kv_head, head_dim, wk, eps);

    if (freq_scale == 1.0f)
        oracle_inv_freq(theta, head_dim, inv);
    else
        oracle_inv_freq_scaled(theta, freq_scale, head_dim, inv);
    if (rope_style == 0) {
        oracle_rope_neox(q, nt, ld_q, n_head, head_dim, pos, inv);
        oracle_rope_neox(k, nt, ld_k, n_kv_head, head_dim, pos, inv);
    } else {
        oracle_rope_interleaved(q, nt, ld_q, n_head, head_dim, pos, inv);
        oracle_rope_interleaved(k, nt, ld_k, n_kv_head, head_dim, pos, inv);
    }

    int64_t bad = oracle_store_rows(k, nt, ld_k, nkt, pos, slot, n_ctx,
                                    n_slots, cache_dtype, row_ids, krows);
    oracle_store_rows(v, nt, ld_v, nkt, pos, slot, n_ctx, n_slots,
                      cache_dtype, row_ids, vrows);
    return bad;
}
