/*
 * oracle.h -- plain f64 CPU oracle for HeadPrep and scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the checker that the GPU library is
 * compared against.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may load it.  It shares no code, header, table or helper with
 * the GPU library, and the GPU library never calls it.
 *
 * Everything is f64 and follows the plain definitions:
 *   - HeadPrep: gizml:netops reference page, "Types > HeadPrep" (split halves, and
 *     FLUX.3's adjacent pairs);
 *   - the whole-row norm and rotary: same page, "Functions > rowNormRopeInto".
 *   - attention, causal mask: gizml:netops reference page, "Functions > attention"
 *     and "Functions > causalMask".
 *   - the quantised KV cache's coding: compute guide "Tensors, GPU kernels and AI
 *     models", Step 5: Run a language model (8, 4 or 2 bits over a least-squared-error
 *     range; decisions in f32).
 * Layouts are row-major, token rows with heads contiguous inside a row.
 * Every function returns 0 on success and a negative value on a bad argument
 * (nothing is written in that case).
 */
#ifndef ATTN_ORACLE_H
#define ATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * HeadPrep, in place, on x laid out [rows, heads, d].
 *   Each head of each row: divide by sqrt(mean of squares + eps), multiply by w[e],
 *   then for e < half turn the pair (e, e + half) by the angle whose cosine and sine
 *   are cos_t[pos[row] * half + e], sin_t[pos[row] * half + e].  Values e >= 2*half
 *   keep their normalised, weighted value.  half == 0 means no rotation.
 *   w: [d]; cos_t, sin_t: [table_rows, half]; pos: [rows] table rows.
 * Returns -1 on a bad size, -2 if a position lies outside [0, table_rows).
 */
int oracle_headprep(double *x, int64_t rows, int64_t heads, int64_t d,
                    const double *w, const double *cos_t, const double *sin_t,
                    int64_t half, int64_t table_rows, const int64_t *pos, double eps);

/*
 * HeadPrep with the turned values as adjacent pairs (FLUX.3's layout, "even values
 * first"): pair (2i, 2i+1), i < half, turns by table entry i of the row; values from
 * 2*half on keep their normalised, weighted value.  Arguments as oracle_headprep.
 */
int oracle_headprep_pairs(double *x, int64_t rows, int64_t heads, int64_t d,
                          const double *w, const double *cos_t, const double *sin_t,
                          int64_t half, int64_t table_rows, const int64_t *pos, double eps);

/*
 * LTX's whole-row norm and rotary, in place on x [rows, width] (width a multiple of
 * head, head even): each row over the RMS of its width values (eps inside the root),
 * times w[e]; then, if cos_t and sin_t are given ([table_rows, width/2], row pos[row]),
 * value j < head/2 of each head h turned with value j + head/2 by pair h*head/2 + j.
 * Returns -1 on a bad size, -2 if a position lies outside [0, table_rows).
 */
int oracle_row_norm_rope(double *x, int64_t rows, int64_t width, int64_t head, const double *w,
                         const double *cos_t, const double *sin_t, int64_t table_rows,
                         const int64_t *pos, double eps);

/*
 * Scaled-dot-product attention, plain definition.
 *   q [batch, tq, hq, d], k [batch, tk, hkv, d], v [batch, tk, hkv, dv] -> out [batch, tq, hq, dv].
 *   q head h reads kv head h / (hq / hkv).
 *   Keys visible to query i of sequence b: j < n_b, where n_b = lens ? lens[b] : tk,
 *   and, when causal, j <= i + n_b - tq (bottom-right alignment).
 *   out = sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s), s_j = scale * q.k_j.
 *   A query with no visible key gets an all-zero output row.
 * Returns -1 on a bad size (hq not a multiple of hkv, lens[b] outside [0, tk], ...).
 */
int oracle_attention(const double *q, const double *k, const double *v, double *out,
                     int64_t batch, int64_t tq, int64_t tk, int64_t hq, int64_t hkv,
                     int64_t d, int64_t dv, double scale, int causal, const int64_t *lens);

/*
 * The same attention, only for the nsel query rows named in sel ([nsel, 3] triples
 * (b, i, h)); out is [nsel, dv].  Used to check very large workloads on a sample.
 */
int oracle_attention_rows(const double *q, const double *k, const double *v, double *out,
                          int64_t batch, int64_t tq, int64_t tk, int64_t hq, int64_t hkv,
                          int64_t d, int64_t dv, double scale, int causal, const int64_t *lens,
                          const int64_t *sel, int64_t nsel);

/*
 * Quantised KV cache coding of `units` heads of d f32 values each (x [units, d]) in
 * `bits` in {8, 4, 2}: codes [units, d] in [0, 2^bits - 1], and per unit lo, step (f32)
 * with value lo + step * code.  Candidate ranges centred on (min + max)/2, half-widths
 * (max - min)/2 * (32 - k)/32 for k = 0..23; the least squared error (summed in f64)
 * wins, the widest on a tie; codes rint((x - lo) * (1/step)) clamped, in f32.
 * k_out (may be NULL) receives the winning k.  Returns -1 on a bad argument.
 */
int oracle_kv_quantize(const float *x, int64_t units, int64_t d, int64_t bits, int32_t *codes,
                       float *lo_out, float *step_out, int32_t *k_out);

/*
 * 8-bit operands of the quantised attention path (netops attentionRows with
 * `quantized`): `units` groups of n f32 values (x [units, n]), one scale per group.
 *   oracle_int8_code: s = amax / 127 (1 if amax = 0), code = clamp(rint(x (1/s)), -127, 127).
 *   oracle_e4m3_code: s = amax / 448 (1 if amax = 0), values = E4M3 rounding (nearest,
 *                     ties to even) of x (1/s), returned as floats (times s gives back x).
 * Returns -1 on a bad argument.
 */
int oracle_int8_code(const float *x, int64_t units, int64_t n, int8_t *codes, float *scale);
int oracle_e4m3_code(const float *x, int64_t units, int64_t n, float *values, float *scale);

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_threads(void);

#ifdef __cplusplus
}
#endif

#endif
