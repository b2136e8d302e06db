/*
 * kvq_oracle.c -- plain, slow, obviously-correct CPU oracle for single-query
 * decode attention over a head-major KV cache (f32 and q8 "2f" caches).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code, header, constant or table with
 * the HIP library.
 *
 * Sources (web pages, cited by page and item):
 *   [P1] cortiq-engine 0.3.4, src/cortiq_engine/kv_cache.rs
 *   [P2] cortiq-engine 0.8.49, src/cortiq_engine/kv_cache.rs (same codec)
 *   [P3] franken_ocr 0.8.0, src/native_engine/rswa.rs
 *
 * Two kinds of arithmetic live here, on purpose:
 *   - ATTENTION is computed from its definition in double precision:
 *       s_p = (q . K[p]) / sqrt(hd),  w = softmax(s),  out = sum_p w_p V[p].
 *     The pages reach exactly this (up to rounding order) with a two-pass
 *     softmax ([P1] LayerKvCache::attend) or an online fold ([P3]
 *     decode_attention_scalar_head + fold); both are re-associations of the
 *     same sums, so the oracle materialises the score row and uses two plain
 *     passes.  For the q8 cache the dequantised values are
 *       K^[p][d] = kq[p][d] * ks[p][d/32] * kcol[d],
 *       V^[p][d] = vq[p][d] * vs[p] * vcol[d]
 *     (the algebra of [P1] attend: score = s_k * <q (.) col_k, k_q>, and the
 *     value pass scales each int8 row by its row scale and the result by
 *     vcol), with every product taken in double.
 *   - The q8_2f CODEC is an encoding with exactly one correct output, defined
 *     by the pages in f32 ([P1] quant_row, freeze_cols, append).  It is
 *     computed here step by step in IEEE single precision: one rounding per
 *     operation, correctly-rounded division and sqrtf, round-half-away-from-
 *     zero (roundf), no fused multiply-add.  The build uses
 *     -ffp-contract=off and no fast-math for this reason.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#pragma STDC FP_CONTRACT OFF

/* Positions appended before the per-channel column field freezes
 * ([P1] const KV_COL_WARMUP). */
#define ORC_COL_WARMUP 64
/* K rows carry one scale per 32 channels ([P1] const KV_K_GROUP); V rows
 * carry one scale per row (group = head_dim). */
#define ORC_K_GROUP 32

int orc_col_warmup(void) { return ORC_COL_WARMUP; }
int orc_k_group(void) { return ORC_K_GROUP; }

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

/* ------------------------------------------------------------------------ */
/* Codec: [P1] LayerKvCache::quant_row.                                      */
/*                                                                            */
/* x[hd]     one f32 row                                                      */
/* col[hd]   per-channel column field, or NULL before the freeze (the pages'  */
/*           "empty col", which divides by nothing)                           */
/* group     elements per scale: 32 for K, hd for V; the last group may be    */
/*           shorter when hd is not a multiple of the group                   */
/* q[hd]     int8 codes out;  s[ceil(hd/group)]  f32 scales out               */
/*                                                                            */
/* Steps: resid = x / col; per group absmax of |resid|;                       */
/* s = max(absmax / 127, 1e-12); code = clamp(round(resid / s), -127, 127)    */
/* with round = half away from zero.                                          */
/* ------------------------------------------------------------------------ */
void orc_quant_row(const float* x, const float* col, int hd, int group,
                   int8_t* q, float* s)
{
    float* resid = (float*)malloc(sizeof(float) * (size_t)hd);
    for (int d = 0; d < hd; ++d) {
        resid[d] = (col == NULL) ? x[d] : x[d] / col[d];
    }
    int gi = 0;
    for (int g0 = 0; g0 < hd; g0 += group, ++gi) {
        int g1 = g0 + group < hd ? g0 + group : hd;
        float absmax = 0.0f;
        for (int d = g0; d < g1; ++d) {
            float a = fabsf(resid[d]);
            if (a > absmax) absmax = a;
        }
        float sc = absmax / 127.0f;
        if (sc < 1e-12f) sc = 1e-12f;
        s[gi] = sc;
        for (int d = g0; d < g1; ++d) {
            float r = roundf(resid[d] / sc);
            if (r < -127.0f) r = -127.0f;
            if (r > 127.0f) r = 127.0f;
            q[d] = (int8_t)r;
        }
    }
    free(resid);
}

/* ------------------------------------------------------------------------ */
/* Codec: [P1] LayerKvCache::freeze_cols, for one head and one of K or V.    */
/*                                                                            */
/* n rows of codes q[n][hd] with scales s[n][ns] (ns = ceil(hd/group)) are    */
/* dequantised (x^ = f32(code) * scale), the column field is the per-channel  */
/* RMS over the n rows,                                                       */
/*     col[d] = max(sqrtf((sum_p x^[p][d]^2) / n), 1e-6),                     */
/* with the sum taken sequentially over p in f32 (multiply, then add), and    */
/* every row is requantised from x^ against col with orc_quant_row.           */
/* q and s are overwritten in place; col[hd] receives the field.             */
/* n == 0 leaves everything untouched and returns 0 (the field stays empty).  */
/* ------------------------------------------------------------------------ */
int orc_freeze_one(int n, int hd, int group, int8_t* q, float* s, float* col)
{
    if (n <= 0) return 0;
    int ns = ceil_div(hd, group);
    float* rows = (float*)malloc(sizeof(float) * (size_t)n * (size_t)hd);
    for (int p = 0; p < n; ++p) {
        for (int d = 0; d < hd; ++d) {
            rows[(size_t)p * hd + d] =
                (float)q[(size_t)p * hd + d] * s[(size_t)p * ns + d / group];
        }
    }
    for (int d = 0; d < hd; ++d) col[d] = 0.0f;
    for (int p = 0; p < n; ++p) {
        for (int d = 0; d < hd; ++d) {
            float x = rows[(size_t)p * hd + d];
            float sq = x * x;
            col[d] = col[d] + sq;
        }
    }
    for (int d = 0; d < hd; ++d) {
        float c = sqrtf(col[d] / (float)n);
        col[d] = c > 1e-6f ? c : 1e-6f;
    }
    for (int p = 0; p < n; ++p) {
        orc_quant_row(rows + (size_t)p * hd, col, hd, group,
                      q + (size_t)p * hd, s + (size_t)p * ns);
    }
    free(rows);
    return 1;
}

/* ------------------------------------------------------------------------ */
/* Codec: [P1] LayerKvCache::append for one live head of one sequence, one    */
/* row at a time.  State of the head (caller-owned arrays sized for `cap`):   */
/*   kq[cap][hd], ks[cap][ceil(hd/32)], vq[cap][hd], vs[cap],                 */
/*   kcol[hd], vcol[hd], *n (rows stored), *frozen (0/1).                     */
/* For each new row: if n >= 64 and the field is not frozen yet, freeze it    */
/* first (K with group 32, V with group hd; the freeze happens at the START  */
/* of the append, so rows 0..63 are requantised and row 64 is the first one   */
/* quantised against the frozen field); then quantise the row (K group 32,    */
/* V group hd) against the field, or against nothing before the freeze.       */
/* k_rows / v_rows: [n_new][row_stride] with the head's hd values at offset 0 */
/* of each row.  Returns 0, or -1 if the capacity would be exceeded (nothing  */
/* is written in that case).                                                  */
/* ------------------------------------------------------------------------ */
int orc_q8_append_head(int hd, int cap, int n_new,
                       const float* k_rows, const float* v_rows, int row_stride,
                       int8_t* kq, float* ks, int8_t* vq, float* vs,
                       float* kcol, float* vcol, int* n, int* frozen)
{
    if (*n + n_new > cap) return -1;
    int ngk = ceil_div(hd, ORC_K_GROUP);
    for (int i = 0; i < n_new; ++i) {
        if (*n >= ORC_COL_WARMUP && !*frozen) {
            orc_freeze_one(*n, hd, ORC_K_GROUP, kq, ks, kcol);
            orc_freeze_one(*n, hd, hd, vq, vs, vcol);
            *frozen = 1;
        }
        int p = *n;
        orc_quant_row(k_rows + (size_t)i * row_stride, *frozen ? kcol : NULL,
                      hd, ORC_K_GROUP, kq + (size_t)p * hd, ks + (size_t)p * ngk);
        orc_quant_row(v_rows + (size_t)i * row_stride, *frozen ? vcol : NULL,
                      hd, hd, vq + (size_t)p * hd, vs + p);
        *n = p + 1;
    }
    return 0;
}

/* Explicit freeze of one head ([P1] freeze_cols invoked on demand): no-op when
 * already frozen or when nothing is stored. */
int orc_q8_freeze_head(int hd, int8_t* kq, float* ks, int8_t* vq, float* vs,
                       float* kcol, float* vcol, int n, int* frozen)
{
    if (*frozen || n == 0) return 0;
    orc_freeze_one(n, hd, ORC_K_GROUP, kq, ks, kcol);
    orc_freeze_one(n, hd, hd, vq, vs, vcol);
    *frozen = 1;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* Attention, by definition, in double precision.                            */
/*                                                                            */
/* One KV row set of n rows and hpk query heads that share it (a GQA group;  */
/* [P1] attend_group: Q head h reads KV head h / hpk).                        */
/*   q[hpk][hd]   f32 queries                                                 */
/*   out[hpk][hd] double results; n == 0 gives zeros ([P1] attend_group:      */
/*                "stored == 0 -> out = 0").                                  */
/* score  s[p] = (sum_d q[d] * K^[p][d]) / sqrt(hd)                           */
/* weight w[p] = exp(s[p] - max s) / sum_p' exp(s[p'] - max s)                */
/* output o[d] = sum_p w[p] * V^[p][d]                                        */
/* ------------------------------------------------------------------------ */
typedef double (*orc_elem_fn)(const void* ctx, int p, int d);

typedef struct {
    const float* rows; int hd;
} orc_f32_rows;

static double f32_elem(const void* ctx, int p, int d)
{
    const orc_f32_rows* r = (const orc_f32_rows*)ctx;
    return (double)r->rows[(size_t)p * r->hd + d];
}

typedef struct {
    const int8_t* codes; const float* scales; const float* col;
    int hd; int group; int ns;
} orc_q8_rows;

/* K^[p][d] = code * scale(group of d) * col[d]; col == NULL means 1. */
static double q8_elem(const void* ctx, int p, int d)
{
    const orc_q8_rows* r = (const orc_q8_rows*)ctx;
    double x = (double)r->codes[(size_t)p * r->hd + d]
             * (double)r->scales[(size_t)p * r->ns + d / r->group];
    if (r->col != NULL) x = x * (double)r->col[d];
    return x;
}

/* Beyond the plain definition, [P2] LayerKvCache::attend_group_upto takes:
 *   first    only rows [first, n) are visible; first is clamped to n - 1, so
 *            at least one row is (rows before it get probability 0);
 *   softcap  > 0: the scaled scores are soft-capped (Gemma-2),
 *            s = softcap * tanh(s / softcap); 0 leaves them as they are;
 *   sinks    NULL, or one learned logit per head, treated as one more
 *            score with no value row: the max is taken over it too, and its
 *            exponential enters the normaliser only; it is not capped.     */
static void attend_generic(int n, int hd, int hpk, const float* q,
                           orc_elem_fn kf, const void* kctx,
                           orc_elem_fn vf, const void* vctx,
                           int first, double softcap, const float* sinks, double* out)
{
    for (int i = 0; i < hpk * hd; ++i) out[i] = 0.0;
    if (n <= 0) return;
    if (first > n - 1) first = n - 1;
    if (first < 0) first = 0;
    double scale = 1.0 / sqrt((double)hd);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    for (int h = 0; h < hpk; ++h) {
        const float* qh = q + (size_t)h * hd;
        double* oh = out + (size_t)h * hd;
        for (int p = first; p < n; ++p) {
            double dot = 0.0;
            for (int d = 0; d < hd; ++d) dot += (double)qh[d] * kf(kctx, p, d);
            s[p] = dot * scale;
            if (softcap > 0.0) s[p] = softcap * tanh(s[p] / softcap);
        }
        double m = s[first];
        for (int p = first + 1; p < n; ++p) if (s[p] > m) m = s[p];
        if (sinks != NULL && (double)sinks[h] > m) m = (double)sinks[h];
        double z = 0.0;
        for (int p = first; p < n; ++p) { s[p] = exp(s[p] - m); z += s[p]; }
        if (sinks != NULL) z += exp((double)sinks[h] - m);
        for (int p = first; p < n; ++p) {
            double w = s[p] / z;
            for (int d = 0; d < hd; ++d) oh[d] += w * vf(vctx, p, d);
        }
    }
    free(s);
}

/* f32 rows: k[n][hd], v[n][hd]. */
void orc_attend_f32_ex(int n, int hd, int hpk, const float* q,
                       const float* k, const float* v,
                       int first, double softcap, const float* sinks, double* out)
{
    orc_f32_rows kc = { k, hd };
    orc_f32_rows vc = { v, hd };
    attend_generic(n, hd, hpk, q, f32_elem, &kc, f32_elem, &vc, first, softcap, sinks, out);
}

void orc_attend_f32(int n, int hd, int hpk, const float* q,
                    const float* k, const float* v, double* out)
{
    orc_attend_f32_ex(n, hd, hpk, q, k, v, 0, 0.0, NULL, out);
}

/* q8 rows: kq[n][hd], ks[n][ceil(hd/32)], vq[n][hd], vs[n]; kcol/vcol [hd] or
 * NULL (not frozen). */
void orc_attend_q8_ex(int n, int hd, int hpk, const float* q,
                      const int8_t* kq, const float* ks, const float* kcol,
                      const int8_t* vq, const float* vs, const float* vcol,
                      int first, double softcap, const float* sinks, double* out)
{
    orc_q8_rows kc = { kq, ks, kcol, hd, ORC_K_GROUP, ceil_div(hd, ORC_K_GROUP) };
    orc_q8_rows vc = { vq, vs, vcol, hd, hd, 1 };
    attend_generic(n, hd, hpk, q, q8_elem, &kc, q8_elem, &vc, first, softcap, sinks, out);
}

void orc_attend_q8(int n, int hd, int hpk, const float* q,
                   const int8_t* kq, const float* ks, const float* kcol,
                   const int8_t* vq, const float* vs, const float* vcol,
                   double* out)
{
    orc_attend_q8_ex(n, hd, hpk, q, kq, ks, kcol, vq, vs, vcol, 0, 0.0, NULL, out);
}

/* ------------------------------------------------------------------------ */
/* Per-row int8 route: [P3] quantize_row_i8 and decode_attention_int8.       */
/*                                                                            */
/* quantize_row_i8: maxabs = max |x| over the row (f32); scale = maxabs / 127 */
/* (correctly rounded division), or 1 for an all-zero row; code = clamp(      */
/* round_ties_even(x / scale), -127, 127).  Returns the scale.                */
/* ------------------------------------------------------------------------ */
float orc_quant_row_i8(const float* x, int hd, int8_t* q)
{
    float maxabs = 0.0f;
    for (int d = 0; d < hd; ++d) {
        float a = fabsf(x[d]);
        if (a > maxabs) maxabs = a;
    }
    float scale = maxabs > 0.0f ? maxabs / 127.0f : 1.0f;
    for (int d = 0; d < hd; ++d) {
        float r = rintf(x[d] / scale);          /* default rounding mode: ties to even */
        if (r < -127.0f) r = -127.0f;
        if (r > 127.0f) r = 127.0f;
        q[d] = (int8_t)r;
    }
    return scale;
}

/* quantize_row_i8 over n rows x[n][hd] -> q[n][hd], s[n]. */
void orc_quant_rows_i8(int n, int hd, const float* x, int8_t* q, float* s)
{
    for (int p = 0; p < n; ++p)
        s[p] = orc_quant_row_i8(x + (size_t)p * hd, hd, q + (size_t)p * hd);
}

/* decode_attention_int8 for one KV head: every query head is quantised with
 * quantize_row_i8; its score against row p is the exact integer dot of the
 * codes times qscale * kscale[p] / sqrt(hd); weights by the softmax; the
 * output sums weight * vscale[p] * vcode[p][d] (all in double).
 *   kq[n][hd], ks[n], vq[n][hd], vs[n];  q[hpk][hd];  out[hpk][hd]
 * first and sinks as attend_generic (the visible-row start and a value-less
 * logit per head of [P2] attend_group_upto; 0 and NULL for the page's int8
 * route, which has neither).                                               */
void orc_attend_i8_ex(int n, int hd, int hpk, const float* q,
                      const int8_t* kq, const float* ks, const int8_t* vq, const float* vs,
                      int first, const float* sinks, double* out)
{
    for (int i = 0; i < hpk * hd; ++i) out[i] = 0.0;
    if (n <= 0) return;
    if (first > n - 1) first = n - 1;
    if (first < 0) first = 0;
    int8_t* qc = (int8_t*)malloc((size_t)hd);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double scale = 1.0 / sqrt((double)hd);
    for (int h = 0; h < hpk; ++h) {
        float qs = orc_quant_row_i8(q + (size_t)h * hd, hd, qc);
        double* oh = out + (size_t)h * hd;
        for (int p = first; p < n; ++p) {
            long dot = 0;
            for (int d = 0; d < hd; ++d) dot += (long)qc[d] * (long)kq[(size_t)p * hd + d];
            s[p] = (double)dot * (double)qs * (double)ks[p] * scale;
        }
        double m = s[first];
        for (int p = first + 1; p < n; ++p) if (s[p] > m) m = s[p];
        if (sinks != NULL && (double)sinks[h] > m) m = (double)sinks[h];
        double z = 0.0;
        for (int p = first; p < n; ++p) { s[p] = exp(s[p] - m); z += s[p]; }
        if (sinks != NULL) z += exp((double)sinks[h] - m);
        for (int p = first; p < n; ++p) {
            double w = s[p] / z * (double)vs[p];
            for (int d = 0; d < hd; ++d) oh[d] += w * (double)vq[(size_t)p * hd + d];
        }
    }
    free(s);
    free(qc);
}

void orc_attend_i8(int n, int hd, int hpk, const float* q,
                   const int8_t* kq, const float* ks, const int8_t* vq, const float* vs,
                   double* out)
{
    orc_attend_i8_ex(n, hd, hpk, q, kq, ks, vq, vs, 0, NULL, out);
}

/* Attention weights alone (for the sum-to-one invariant): w[n] for one query
 * head over f32 rows. */
void orc_weights_f32(int n, int hd, const float* q, const float* k, double* w)
{
    if (n <= 0) return;
    double scale = 1.0 / sqrt((double)hd);
    for (int p = 0; p < n; ++p) {
        double dot = 0.0;
        for (int d = 0; d < hd; ++d)
            dot += (double)q[d] * (double)k[(size_t)p * hd + d];
        w[p] = dot * scale;
    }
    double m = w[0];
    for (int p = 1; p < n; ++p) if (w[p] > m) m = w[p];
    double z = 0.0;
    for (int p = 0; p < n; ++p) { w[p] = exp(w[p] - m); z += w[p]; }
    for (int p = 0; p < n; ++p) w[p] = w[p] / z;
}
