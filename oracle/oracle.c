/*
 * oracle.c -- plain f64 CPU oracle for HeadPrep and scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY: the checker the GPU library is compared against.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg load it.  It
 * shares no code with the GPU library.  Loops are plain and unblocked so that each
 * step can be read against the definition it follows; the only parallelism is an
 * OpenMP loop over independent (row, head) or (query row, head) items.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC oracle.c -lm  (no fast-math and
 * no fused multiply-add: IEEE f64, and f32 where a quantised code is decided).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * HeadPrep of one head of d values (gizml:netops reference page, Types > HeadPrep):
 *   1. the head over its RMS, with eps inside the root: x_e / sqrt(mean(x^2) + eps)
 *      (the same eps placement as layerNorm's sqrt(var + eps) on that page);
 *   2. times its norm weight w_e;
 *   3. values e < half turned with e + half by the row's cos and sin (split halves):
 *        a' = a cos - b sin,  b' = b cos + a sin,  with a = x_e, b = x_{e+half};
 *      values from 2*half on are left as they are; half = 0 means no turn.
 */
static void prep_one_head(double *x, int64_t d, const double *w,
                          const double *cos_row, const double *sin_row, int64_t half,
                          double eps)
{
    double ms = 0.0;
    for (int64_t e = 0; e < d; ++e)
        ms += x[e] * x[e];
    ms /= (double)d;
    const double root = sqrt(ms + eps);
    for (int64_t e = 0; e < d; ++e)
        x[e] = x[e] / root * w[e];
    for (int64_t e = 0; e < half; ++e) {
        const double a = x[e], b = x[e + half];
        const double c = cos_row[e], s = sin_row[e];
        x[e] = a * c - b * s;
        x[e + half] = b * c + a * s;
    }
}

int oracle_headprep(double *x, int64_t rows, int64_t heads, int64_t d,
                    const double *w, const double *cos_t, const double *sin_t,
                    int64_t half, int64_t table_rows, const int64_t *pos, double eps)
{
    if (!x || !w || rows < 0 || heads < 0 || d <= 0 || half < 0 || 2 * half > d || eps < 0)
        return -1;
    if (half > 0) {
        if (!cos_t || !sin_t || !pos || table_rows <= 0)
            return -1;
        for (int64_t r = 0; r < rows; ++r)
            if (pos[r] < 0 || pos[r] >= table_rows)
                return -2;
    }
#pragma omp parallel for schedule(static)
    for (int64_t item = 0; item < rows * heads; ++item) {
        const int64_t r = item / heads;
        const double *c = half > 0 ? cos_t + pos[r] * half : NULL;
        const double *s = half > 0 ? sin_t + pos[r] * half : NULL;
        prep_one_head(x + item * d, d, w, c, s, half, eps);
    }
    return 0;
}

/*
 * One output row of attention (gizml:netops reference page, Functions > attention,
 * and Functions > causalMask for the visible keys):
 *   s_j = scale * sum_p q_p k_jp for each visible key j, m = max_j s_j,
 *   out = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m).
 * Visible keys: j < n, and j <= i + n - tq when causal.  No visible key: zeros.
 * s is scratch of at least n doubles.
 */
/*
 * The same HeadPrep with the turned values taken as adjacent pairs (gizml:netops
 * reference page, Types > HeadPrep: FLUX.3's pairs, loaded even values first): the
 * head's values are read even ones first, so value 2i plays the part of value i and
 * value 2i + 1 that of value i + half.  Pair (2i, 2i + 1), i < half, turns by table
 * entry i:  a' = a cos - b sin,  b' = b cos + a sin,  a = x_{2i},  b = x_{2i+1}.
 * Values from 2*half on are left as they are.
 */
static void prep_one_head_pairs(double *x, int64_t d, const double *w,
                                const double *cos_row, const double *sin_row, int64_t half,
                                double eps)
{
    double sq = 0.0;
    for (int64_t e = 0; e < d; ++e)
        sq += x[e] * x[e];
    const double rt = sqrt(sq / (double)d + eps);
    for (int64_t e = 0; e < d; ++e)
        x[e] = x[e] * w[e] / rt;
    for (int64_t i = 0; i < half; ++i) {
        const double a = x[2 * i], b = x[2 * i + 1];
        const double c = cos_row[i], s = sin_row[i];
        x[2 * i] = a * c - b * s;
        x[2 * i + 1] = b * c + a * s;
    }
}

int oracle_headprep_pairs(double *x, int64_t rows, int64_t heads, int64_t d,
                          const double *w, const double *cos_t, const double *sin_t,
                          int64_t half, int64_t table_rows, const int64_t *pos, double eps)
{
    if (!x || !w || rows < 0 || heads < 0 || d <= 0 || half < 0 || 2 * half > d || eps < 0)
        return -1;
    if (half > 0) {
        if (!cos_t || !sin_t || !pos || table_rows <= 0)
            return -1;
        for (int64_t r = 0; r < rows; ++r)
            if (pos[r] < 0 || pos[r] >= table_rows)
                return -2;
    }
#pragma omp parallel for schedule(static)
    for (int64_t item = 0; item < rows * heads; ++item) {
        const int64_t r = item / heads;
        const double *c = half > 0 ? cos_t + half * pos[r] : NULL;
        const double *s = half > 0 ? sin_t + half * pos[r] : NULL;
        prep_one_head_pairs(x + item * d, d, w, c, s, half, eps);
    }
    return 0;
}

/*
 * The whole-row norm and rotary of LTX (gizml:netops reference page, Functions >
 * rowNormRopeInto), in place on x [rows, width]:
 *   1. each row over the RMS of all its width values, eps inside the root, times w[e];
 *   2. with tables (cos_t, sin_t [table_rows, width/2]): each head of `head` values
 *      turned by split halves, value j < head/2 of head h with value j + head/2 by
 *      the angle of pair h*head/2 + j of the row's table row pos[row].
 */
int oracle_row_norm_rope(double *x, int64_t rows, int64_t width, int64_t head, const double *w,
                         const double *cos_t, const double *sin_t, int64_t table_rows,
                         const int64_t *pos, double eps)
{
    if (!x || !w || rows < 0 || width <= 0 || head <= 0 || head % 2 != 0 || width % head != 0 || eps < 0)
        return -1;
    if (cos_t || sin_t) {
        if (!cos_t || !sin_t || !pos || table_rows <= 0)
            return -1;
        for (int64_t r = 0; r < rows; ++r)
            if (pos[r] < 0 || pos[r] >= table_rows)
                return -2;
    }
    const int64_t half = head / 2, tw = width / 2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double *xr = x + r * width;
        double acc = 0.0;
        for (int64_t e = 0; e < width; ++e)
            acc += xr[e] * xr[e];
        acc /= (double)width;
        const double nrm = sqrt(acc + eps);
        for (int64_t e = 0; e < width; ++e)
            xr[e] = xr[e] * w[e] / nrm;
        if (!cos_t)
            continue;
        const double *c = cos_t + pos[r] * tw, *s = sin_t + pos[r] * tw;
        for (int64_t h = 0; h < width / head; ++h)
            for (int64_t j = 0; j < half; ++j) {
                const int64_t ia = h * head + j, ib = ia + half, t = h * half + j;
                const double a = xr[ia], b = xr[ib];
                xr[ia] = a * c[t] - b * s[t];
                xr[ib] = b * c[t] + a * s[t];
            }
    }
    return 0;
}

/*
 * Coding of a quantised KV cache (compute guide "Tensors, GPU kernels and AI models",
 * Step 5: Run a language model -- keys and values kept in 8, 4 or 2 bits, each head coded
 * over the range that returns it with the least squared error).  One unit is one head of one token: d float values.  With L = 2^bits levels,
 * a range [lo, lo + (L-1) step] gives value x the code rint((x - lo) / step) clamped to
 * [0, L-1], and back the value lo + step code.  The candidate ranges are centred on
 * (min + max)/2 with half-widths r (32 - k)/32, k = 0..23 (r = (max - min)/2); the
 * candidate giving the least squared error wins, the widest on a tie.  Every step that
 * decides a code runs in f32, in the order written (the division as a product with the
 * f32 reciprocal of step); the squared error of a candidate is summed in f64.  A unit
 * whose half-range r is 1e-30 or less is coded as lo = min, step = 0, codes 0.
 */
/* Candidate k of a unit with half-range r around centre: its lo, step and 1/step. */
static void kv_candidate(float centre, float r, int32_t k, int32_t top, float *lo, float *st, float *inv)
{
    const float hw = r * ((float)(32 - k) / 32.0f);
    *lo = centre - hw;
    *st = (hw + hw) / (float)top;
    *inv = 1.0f / *st;
}

/* The code of value x in the range (lo, 1/step): nearest level, clamped to [0, top]. */
static int32_t kv_code(float x, float lo, float inv, int32_t top)
{
    float t = rintf((x - lo) * inv);
    if (t < 0.0f) t = 0.0f;
    if (t > (float)top) t = (float)top;
    return (int32_t)t;
}

int oracle_kv_quantize(const float *x, int64_t units, int64_t d, int64_t bits, int32_t *codes,
                       float *lo_out, float *step_out, int32_t *k_out)
{
    if (!x || !codes || !lo_out || !step_out || units < 0 || d <= 0 || (bits != 8 && bits != 4 && bits != 2))
        return -1;
    const int32_t top = (1 << bits) - 1;
#pragma omp parallel for schedule(static)
    for (int64_t u = 0; u < units; ++u) {
        const float *xu = x + u * d;
        int32_t *cu = codes + u * d;
        float mn = xu[0], mx = xu[0];
        for (int64_t e = 1; e < d; ++e) {
            if (xu[e] < mn) mn = xu[e];
            if (xu[e] > mx) mx = xu[e];
        }
        const float centre = (mn + mx) * 0.5f;
        const float r = (mx - mn) * 0.5f;
        if (!(r > 1e-30f)) {
            lo_out[u] = mn;
            step_out[u] = 0.0f;
            for (int64_t e = 0; e < d; ++e) cu[e] = 0;
            if (k_out) k_out[u] = 0;
            continue;
        }
        double best = INFINITY;
        int32_t best_k = 0;
        for (int32_t k = 0; k < 24; ++k) {
            float lo, st, inv;
            kv_candidate(centre, r, k, top, &lo, &st, &inv);
            double sse = 0.0;
            for (int64_t e = 0; e < d; ++e) {
                const double back = (double)lo + (double)st * (double)kv_code(xu[e], lo, inv, top);
                const double err = (double)xu[e] - back;
                sse += err * err;
            }
            if (sse < best) {
                best = sse;
                best_k = k;
            }
        }
        float lo, st, inv;
        kv_candidate(centre, r, best_k, top, &lo, &st, &inv);
        for (int64_t e = 0; e < d; ++e)
            cu[e] = kv_code(xu[e], lo, inv, top);
        lo_out[u] = lo;
        step_out[u] = st;
        if (k_out) k_out[u] = best_k;
    }
    return 0;
}

/*
 * 8-bit operands of the quantised attention path (gizml:netops, Functions >
 * attentionRows: with `quantized`, Q K^T on INT8 and P V on E4M3, SageAttention's split).
 * Each unit of n f32 values shares one scale; every decision runs in f32 as written.
 *   int8: s = amax / 127, code = clamp(rint(x * (1 / s)), -127, 127); amax = 0 gives s = 1,
 *         codes 0.  The unit gives back code * s.
 *   e4m3: s = amax / 448, value = the E4M3 number nearest to x * (1 / s) (ties to the even
 *         code; 3 fraction bits, exponent bias 7, subnormal step 2^-9, largest 448), given
 *         back times s.  amax = 0 gives s = 1, values 0.
 */
int oracle_int8_code(const float *x, int64_t units, int64_t n, int8_t *codes, float *scale)
{
    if (!x || !codes || !scale || units < 0 || n <= 0)
        return -1;
    for (int64_t u = 0; u < units; ++u) {
        const float *xu = x + u * n;
        float amax = 0.0f;
        for (int64_t i = 0; i < n; ++i)
            if (fabsf(xu[i]) > amax) amax = fabsf(xu[i]);
        const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
        const float inv = 1.0f / s;
        for (int64_t i = 0; i < n; ++i) {
            float t = rintf(xu[i] * inv);
            if (t < -127.0f) t = -127.0f;
            if (t > 127.0f) t = 127.0f;
            codes[u * n + i] = (int8_t)t;
        }
        scale[u] = s;
    }
    return 0;
}

/* The E4M3 number nearest to a (ties to even), a finite f32 with |a| <= 464. */
static float e4m3_round(float a)
{
    const float m = fabsf(a);
    float step;
    if (m < 0.015625f) {                      /* below 2^-6: subnormal spacing 2^-9 */
        step = 0.001953125f;
    } else {
        int e;
        frexpf(m, &e);                        /* m = f 2^e, f in [0.5, 1) */
        step = ldexpf(1.0f, e - 1 - 3);       /* 3 fraction bits below the leading one */
    }
    const float q = rintf(m / step) * step;   /* m / step and the product are exact */
    return a < 0.0f ? -q : q;
}

int oracle_e4m3_code(const float *x, int64_t units, int64_t n, float *values, float *scale)
{
    if (!x || !values || !scale || units < 0 || n <= 0)
        return -1;
    for (int64_t u = 0; u < units; ++u) {
        const float *xu = x + u * n;
        float amax = 0.0f;
        for (int64_t i = 0; i < n; ++i)
            if (fabsf(xu[i]) > amax) amax = fabsf(xu[i]);
        const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        const float inv = 1.0f / s;
        for (int64_t i = 0; i < n; ++i)
            values[u * n + i] = e4m3_round(xu[i] * inv);
        scale[u] = s;
    }
    return 0;
}

static void attend_one(const double *q, const double *k, const double *v, double *out,
                       int64_t b, int64_t i, int64_t h,
                       int64_t tq, int64_t tk, int64_t hq, int64_t hkv,
                       int64_t d, int64_t dv, double scale, int causal, int64_t n, double *s)
{
    const int64_t g = h / (hq / hkv);
    const double *qi = q + ((b * tq + i) * hq + h) * d;
    int64_t last = n - 1;                         /* last visible key */
    if (causal && i + n - tq < last)
        last = i + n - tq;
    for (int64_t e = 0; e < dv; ++e)
        out[e] = 0.0;
    if (last < 0)
        return;
    double m = -INFINITY;
    for (int64_t j = 0; j <= last; ++j) {
        const double *kj = k + ((b * tk + j) * hkv + g) * d;
        double dot = 0.0;
        for (int64_t p = 0; p < d; ++p)
            dot += qi[p] * kj[p];
        s[j] = scale * dot;
        if (s[j] > m)
            m = s[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j <= last; ++j) {
        const double wj = exp(s[j] - m);
        const double *vj = v + ((b * tk + j) * hkv + g) * dv;
        sum += wj;
        for (int64_t e = 0; e < dv; ++e)
            out[e] += wj * vj[e];
    }
    for (int64_t e = 0; e < dv; ++e)
        out[e] /= sum;
}

static int check_attention_args(const double *q, const double *k, const double *v,
                                const double *out, int64_t batch, int64_t tq, int64_t tk,
                                int64_t hq, int64_t hkv, int64_t d, int64_t dv,
                                const int64_t *lens)
{
    if (!q || !k || !v || !out)
        return -1;
    if (batch < 0 || tq < 0 || tk < 0 || hq <= 0 || hkv <= 0 || d <= 0 || dv <= 0)
        return -1;
    if (hq % hkv != 0)
        return -1;
    if (lens)
        for (int64_t b = 0; b < batch; ++b)
            if (lens[b] < 0 || lens[b] > tk)
                return -1;
    return 0;
}

int oracle_attention(const double *q, const double *k, const double *v, double *out,
                     int64_t batch, int64_t tq, int64_t tk, int64_t hq, int64_t hkv,
                     int64_t d, int64_t dv, double scale, int causal, const int64_t *lens)
{
    if (check_attention_args(q, k, v, out, batch, tq, tk, hq, hkv, d, dv, lens))
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(tk > 0 ? tk : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t item = 0; item < batch * tq * hq; ++item) {
                const int64_t h = item % hq;
                const int64_t i = (item / hq) % tq;
                const int64_t b = item / (hq * tq);
                const int64_t n = lens ? lens[b] : tk;
                attend_one(q, k, v, out + item * dv, b, i, h, tq, tk, hq, hkv, d, dv,
                           scale, causal, n, s);
            }
        }
        free(s);
    }
    return bad ? -3 : 0;
}

int oracle_attention_rows(const double *q, const double *k, const double *v, double *out,
                          int64_t batch, int64_t tq, int64_t tk, int64_t hq, int64_t hkv,
                          int64_t d, int64_t dv, double scale, int causal, const int64_t *lens,
                          const int64_t *sel, int64_t nsel)
{
    if (check_attention_args(q, k, v, out, batch, tq, tk, hq, hkv, d, dv, lens))
        return -1;
    if (nsel < 0 || (nsel > 0 && !sel))
        return -1;
    for (int64_t r = 0; r < nsel; ++r) {
        const int64_t b = sel[3 * r], i = sel[3 * r + 1], h = sel[3 * r + 2];
        if (b < 0 || b >= batch || i < 0 || i >= tq || h < 0 || h >= hq)
            return -1;
    }
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(tk > 0 ? tk : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < nsel; ++r) {
                const int64_t b = sel[3 * r], i = sel[3 * r + 1], h = sel[3 * r + 2];
                const int64_t n = lens ? lens[b] : tk;
                attend_one(q, k, v, out + r * dv, b, i, h, tq, tk, hq, hkv, d, dv,
                           scale, causal, n, s);
            }
        }
        free(s);
    }
    return bad ? -3 : 0;
}
