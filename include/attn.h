/*
 * attn.h -- C ABI of libattn: HeadPrep and scaled-dot-product attention (causal
 * prefill, single-row decode against a KV cache, grouped K/V heads) on AMD
 * MI355X (gfx950).
 *
 * What is computed (gizml:netops reference page):
 *   - HeadPrep (Types > HeadPrep): each head of q and k is divided by
 *     sqrt(mean of its squares + eps), multiplied by its norm weight (qw for q,
 *     kw for k: one [d] f32 vector shared by every head), then every value e < half
 *     is turned with value e + half by the cosine and sine of its row:
 *         a' = a cos - b sin,   b' = b cos + a sin   (a = x[e], b = x[e + half]).
 *     Values from 2*half on keep their normed, weighted value; half = 0: no turn.
 *   - The cos/sin row of a token is its sequence position (Functions >
 *     headPrepInPlace: row0 is the sequence row of the first row).
 *   - attention (Functions > attention, Functions > causalMask):
 *         out = softmax(q k^T * scale [+ mask]) v,
 *     where with causal query i sees key j iff j <= i + tk - tq.  The (tq, tk)
 *     score matrix is never stored.
 *   - Grouped K/V heads: q head h reads kv head h / (hq / hkv); hkv divides hq.
 *   - Output type is the operand type; sums run in f32 and are rounded once, to
 *     nearest even, at the end (compute internals page, "Tensor cores": the product
 *     type is the operands' type).
 *
 * Layout: row-major, token rows with heads contiguous inside a row: element
 * (b, t, h, e) of a [batch, seq, heads, d] tensor with row stride rs (elements
 * between consecutive tokens, rs >= heads * d) is at ((b * seq + t) * rs + h * d + e).
 * A packed qkv buffer [n, (hq + 2 hkv) d] is described by three pointers into it
 * with the same row stride.
 *
 * Ownership: every pointer is caller-owned device memory (HIP device allocations on
 * the current device).  The library allocates nothing, keeps no per-call state and
 * never synchronises: work is enqueued on `stream` (a hipStream_t; NULL is the null
 * stream) and the call returns.  Inputs must stay valid until that work has run.
 *
 * Errors: every argument is checked on the host before anything is enqueued; a call
 * that returns an error has enqueued nothing (it fails closed).  The message of the
 * last failure on the calling thread is available from attn_last_error().
 *   ATTN_ERR_ARG          null pointer, size < 0, hq % hkv != 0, 2*half > d, a row
 *                         stride smaller than its row, positions past the table,
 *                         scale <= 0, ...  (batch or seq 0 is a no-op returning ATTN_OK)
 *   ATTN_ERR_UNSUPPORTED  head dim d not in {64, 128}, or an unknown dtype.
 *   ATTN_ERR_WORKSPACE    decode workspace smaller than attn_decode_workspace_size().
 *   ATTN_ERR_HIP          the HIP runtime reported an error while enqueuing.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_dtype {
    ATTN_F32 = 0,   /* IEEE binary32 operands */
    ATTN_BF16 = 1   /* bfloat16 operands (f32 accumulation) */
} attn_dtype_t;

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_ARG = -1,
    ATTN_ERR_UNSUPPORTED = -2,
    ATTN_ERR_WORKSPACE = -3,
    ATTN_ERR_HIP = -4
} attn_status_t;

/*
 * The HeadPrep record (gizml:netops, Types > HeadPrep: {qw, kw, cos, sin, eps}).
 * All pointers are device f32 arrays.
 *   qw, kw      [d] norm weights of q and of k.
 *   cos, sin    [table_rows, half] rotation tables; row p is sequence position p.
 *   half        number of turned pairs; 0 <= 2 * half <= d; 0 means no turn (cos and
 *               sin are then not read and may be NULL).
 *   table_rows  number of rows in cos and sin; every position used must be below it.
 *   eps         added to the mean of squares under the root (taken as f32).
 *   pairs       which values turn together with table entry i < half:
 *                 0  split halves: value i with value i + half (the HeadPrep above);
 *                 1  adjacent pairs: value 2i with value 2i + 1, the even value
 *                    playing a and the odd b (FLUX.3's rotary, gizml:netops, Types >
 *                    HeadPrep: loaded with its even values first, a head turns as
 *                    split halves; pairs = 1 takes the head as stored, interleaved).
 *               Values from 2 * half on keep their normed, weighted value either way.
 *   kmax        0, or a bound the caller guarantees on the L2 norm of every key row
 *               the attention reads (as stored, after its HeadPrep); finite, >= 0.
 *               attn_key_bound gives the bound HeadPrep with weights kw guarantees.
 *               With a bound (kmax, or kw when the call preps k itself), the bf16
 *               prefill with q's HeadPrep fused shifts each query row's softmax by
 *               |q| times the bound (which no score of the row can exceed) instead of
 *               tracking a running maximum: the same softmax, in fewer instructions
 *               per key tile.  Rows whose shift would exceed 48 (in log2 units) keep
 *               the running maximum.  An understated kmax can overflow the weights.
 *               The bound derived from kw assumes cos and sin tables that turn: cos^2 +
 *               sin^2 <= 1 at every entry (up to f32 rounding); with other tables give
 *               kmax = 0 or a bound of your own.
 *               Other entry points ignore it.
 *               A zero-initialised record is the split-halves HeadPrep with no bound.
 */
typedef struct attn_headprep {
    const float *qw;
    const float *kw;
    const float *cos;
    const float *sin;
    int64_t half;
    int64_t table_rows;
    double eps;
    int64_t pairs;
    double kmax;
} attn_headprep_t;

/*
 * attn_key_bound -- the bound on the norm of every key row that HeadPrep with norm
 * weights kw writes, for attn_headprep_t.kmax: sqrt(d) max|kw| (an RMS-normed row
 * has norm at most sqrt(d), the weights scale it by at most max|kw|, the turn keeps
 * it) times 1 + 2^-7 (rounding to bf16 changes each value by at most 2^-9 of it).
 *   kw  HOST pointer to d floats.  Returns -1 if kw is NULL or d <= 0, NaN if a
 *   weight is not finite.
 */
double attn_key_bound(const float *kw, int64_t d);

/*
 * attn_prep -- HeadPrep in place on q and k (gizml:netops, Functions >
 * headPrepInPlace).
 *   q  [batch, seq, hq, d], row stride q_row_stride; prepped with qw.  May be NULL.
 *   k  [batch, seq, hkv, d], row stride k_row_stride; prepped with kw.  May be NULL.
 *   Token t of every sequence uses table row pos0 + t; pos0 + seq <= table_rows.
 *   dtype is the storage type of q and k; the arithmetic is f32 and the result is
 *   rounded once to the storage type.  hq (hkv) is ignored when q (k) is NULL.
 */
attn_status_t attn_prep(void *q, void *k, int64_t batch, int64_t seq, int64_t hq, int64_t hkv,
                        int64_t d, int64_t q_row_stride, int64_t k_row_stride, int64_t pos0,
                        const attn_headprep_t *prep, attn_dtype_t dtype, void *stream);

/*
 * attn_prefill -- causal (or full) attention of a whole sequence, with HeadPrep.
 *   q    [batch, seq, hq, d]   (read only; its HeadPrep is applied as it is read)
 *   k    [batch, seq, hkv, d]  (with prep: prepped IN PLACE first, so on return it
 *                               holds the prepped keys, ready to serve as a KV cache)
 *   v    [batch, seq, hkv, d]
 *   out  [batch, seq, hq, d]   must not overlap q, k or v.
 *   Token t uses table row pos0 + t.  prep may be NULL: plain attention of q, k, v.
 *   prep->kw may be NULL: k then already holds prepped keys (e.g. written by an
 *   earlier attn_prep) and is not modified; q's HeadPrep is still applied.
 *   causal != 0: query t sees keys 0..t (tq = tk, so bottom-right = top-left).
 *   scale multiplies q.k; finite and > 0 (1/sqrt(d) in the usual model).
 */
attn_status_t attn_prefill(const void *q, void *k, const void *v, void *out,
                           int64_t batch, int64_t seq, int64_t hq, int64_t hkv, int64_t d,
                           int64_t q_row_stride, int64_t k_row_stride, int64_t v_row_stride,
                           int64_t o_row_stride, int64_t pos0, const attn_headprep_t *prep,
                           int causal, double scale, attn_dtype_t dtype, void *stream);

/*
 * attn_prefill_chunk -- a chunk of tq new tokens per sequence against a KV cache that
 * already holds n_past prepped rows (chunked prefill: gizml:netops, Functions >
 * attention with tq < tk, whose causal mask is aligned bottom-right), appending the
 * chunk's keys and values to the cache.  In order, on `stream`:
 *   1. k_cache[b, n_past + t] = HeadPrep of k_new[b, t] at table row n_past + t with kw
 *      (prep NULL or prep->kw NULL: k_new holds prepped keys and is copied as it is);
 *   2. v_cache[b, n_past + t] = v_new[b, t];
 *   3. out[b, i] = attention of q[b, i] (its HeadPrep at table row n_past + i when prep
 *      is given) over cache rows 0 .. n_past + tq - 1; with causal != 0, query i sees
 *      rows j <= n_past + i.
 *   q            [batch, tq, hq, d] contiguous, read only
 *   k_new, v_new [batch, tq, hkv, d] contiguous, read only
 *   k_cache, v_cache [batch, capacity, hkv, d] contiguous; rows 0 .. n_past - 1 must
 *                hold the earlier tokens (keys prepped); rows n_past .. n_past + tq - 1
 *                are overwritten; later rows are not touched.
 *   out          [batch, tq, hq, d] contiguous; must not overlap any other buffer.
 *   n_past       with past NULL, every sequence's cached rows; 0 <= n_past, n_past + tq
 *                <= capacity (n_past = 0 is attn_prefill of the chunk with the cache as
 *                k and v).  With past given, the host bound on every past[b].
 *   past         NULL, or device int32 [batch]: sequence b holds past[b] cached rows and
 *                everything above reads past[b] for n_past for that sequence (one engine
 *                step over sequences at different positions: compute guide "Tensors,
 *                GPU kernels and AI models", Step 5).  A past[b] outside [0, n_past] gives
 *                NaN output rows for sequence b and writes none of its cache rows.  Must
 *                not overlap out or the caches.
 *   scale        finite and > 0.
 *   The caches must not overlap each other or k_new / v_new.  Errors as attn_prefill.
 */
attn_status_t attn_prefill_chunk(const void *q, const void *k_new, const void *v_new, void *k_cache,
                                 void *v_cache, void *out, int64_t batch, int64_t tq, int64_t hq,
                                 int64_t hkv, int64_t d, int64_t capacity, int64_t n_past,
                                 const int32_t *past, const attn_headprep_t *prep, int causal,
                                 double scale, attn_dtype_t dtype, void *stream);

/*
 * attn_prefill_chunk_paged -- attn_prefill_chunk with the cache in a paged KV pool
 * (compute guide "Tensors, GPU kernels and AI models", Step 5): k_pool, v_pool
 * [num_pages, page_rows, hkv, d] and the page table pages [batch, max_pages] (device
 * int32) as in attn_decode_paged, with page_rows a power of two in [64, 2^20].  The
 * chunk's keys (prepped when prep->kw is set) and values are written to rows n_past ..
 * n_past + tq - 1 of each sequence's pages; its queries then attend rows 0 .. n_past +
 * tq - 1 read through the table.  n_past + tq <= max_pages * page_rows.  past as in
 * attn_prefill_chunk (sequence b's rows past[b] .. of its pages; n_past the bound).  A
 * page id outside [0, num_pages) is not written and gives NaN output rows for its
 * sequence.  bf16 only (ATTN_ERR_UNSUPPORTED for f32).
 */
attn_status_t attn_prefill_chunk_paged(const void *q, const void *k_new, const void *v_new, void *k_pool,
                                       void *v_pool, void *out, int64_t batch, int64_t tq, int64_t hq,
                                       int64_t hkv, int64_t d, int64_t num_pages, int64_t page_rows,
                                       const int32_t *pages, int64_t max_pages, int64_t n_past,
                                       const int32_t *past, const attn_headprep_t *prep, int causal,
                                       double scale, attn_dtype_t dtype, void *stream);

/*
 * attn_decode -- one new query row per sequence against a KV cache whose keys are
 * already prepped (gizml:netops, Functions > attention with tq = 1 < tk: the row
 * attends the whole cache).
 *   q         [batch, hq, d] contiguous; its HeadPrep (qw, cos, sin) is applied at
 *             table row pos[b] as it is read; kw is not used.  prep may be NULL.
 *   k_cache   [batch, capacity, hkv, d] contiguous, prepped keys.
 *   v_cache   [batch, capacity, hkv, d] contiguous.
 *   out       [batch, hq, d] contiguous.
 *   lens      device int32 [batch]: sequence b attends cache rows 0 .. lens[b]-1.
 *   pos       device int32 [batch]: table row of sequence b's query (read only when
 *             prep is given and half > 0; may be NULL otherwise).
 *   max_len   host bound on every lens[b]; 1 <= max_len <= capacity.  It sets how
 *             the keys are split.
 *   max_pos   host bound on every pos[b]: with a turning HeadPrep (half > 0),
 *             0 <= max_pos < prep->table_rows is checked before anything is
 *             enqueued (ATTN_ERR_ARG otherwise); without one it is ignored.
 *   splits    number of key splits per sequence, 0 = the library's choice
 *             (attn_decode_default_splits).  Results do not depend on it beyond
 *             rounding.
 *   workspace device scratch of at least attn_decode_workspace_size(...) bytes with
 *             the same batch, hq, hkv, d, max_len and splits.  Contents on entry are
 *             ignored.  Calls that share a workspace must not overlap in time.  The
 *             size is 0 when the call runs as a single split (the output is then
 *             written directly); workspace may be NULL in that case.
 *   Device-side values the host cannot check: lens[b] == 0 gives a zero output row;
 *   lens[b] < 0, lens[b] > max_len, or a pos[b] outside [0, max_pos] gives NaN in
 *   that sequence's output rows (nothing outside the buffers is read).
 */
size_t attn_decode_workspace_size(int64_t batch, int64_t hq, int64_t hkv, int64_t d,
                                  int64_t max_len, int64_t splits);
int64_t attn_decode_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t d, int64_t max_len);
attn_status_t attn_decode(const void *q, const void *k_cache, const void *v_cache, void *out,
                          int64_t batch, int64_t hq, int64_t hkv, int64_t d, int64_t capacity,
                          const int32_t *lens, const int32_t *pos, int64_t max_len, int64_t max_pos,
                          const attn_headprep_t *prep, double scale, int64_t splits,
                          void *workspace, size_t workspace_bytes, attn_dtype_t dtype,
                          void *stream);

/*
 * attn_decode_paged -- attn_decode over a paged KV pool (compute guide "Tensors, GPU
 * kernels and AI models", Step 5: the engine's KV pool, which slots share by reading one
 * copy of a common start's keys and values).  bf16 only.
 *   k_pool, v_pool  [num_pages, page_rows, hkv, d]: each page is laid out as a cache of
 *                   batch 1 and capacity page_rows (attn_prep and plain copies write rows
 *                   into a page in place).
 *   pages           [batch, max_pages] int32, device: key j of sequence b is row
 *                   j % page_rows of page pages[b * max_pages + j / page_rows].  Pages may
 *                   be shared between sequences (a common prefix is read from one copy).
 *   page_rows       a power of two in [16, 2^20]; num_pages * page_rows < 2^31;
 *                   max_len <= max_pages * page_rows.
 *   Everything else is attn_decode's.  A page id outside [0, num_pages) among the pages
 *   a sequence reads gives NaN rows for it (reads stay inside the pool).
 *   ATTN_ERR_UNSUPPORTED for f32.
 */
attn_status_t attn_decode_paged(const void *q, const void *k_pool, const void *v_pool, void *out,
                                int64_t batch, int64_t hq, int64_t hkv, int64_t d, int64_t num_pages,
                                int64_t page_rows, const int32_t *pages, int64_t max_pages,
                                const int32_t *lens, const int32_t *pos, int64_t max_len, int64_t max_pos,
                                const attn_headprep_t *prep, double scale, int64_t splits,
                                void *workspace, size_t workspace_bytes, attn_dtype_t dtype,
                                void *stream);

/*
 * attn_decode_static -- attn_decode without a workspace, for callers that cannot
 * allocate device memory (code under stream or graph capture, tight serving loops,
 * hosts that forbid allocation).  The split partials go to a scratch array of
 * attn_decode_static_scratch_bytes() (8 MiB) that the library holds in device memory,
 * one per device, until the process ends.  This call allocates nothing; its first call
 * on a device looks the array's address up once.
 *   Every argument is attn_decode's.  splits = 0 takes attn_decode_default_splits,
 *   lowered until the partials (splits * batch * hq * (d + 2) * 4 bytes when splits > 1;
 *   none for one split) fit the scratch.  An explicit split count whose partials do not
 *   fit is rejected with ATTN_ERR_WORKSPACE before anything is enqueued.
 *   Every call on one device shares that device's scratch, and nothing in it must start
 *   at zero: calls that overlap in time on one device (other streams, other host
 *   threads) race and give wrong results.  Results equal attn_decode's with the same
 *   split count.
 */
size_t attn_decode_static_scratch_bytes(void);
attn_status_t attn_decode_static(const void *q, const void *k_cache, const void *v_cache, void *out,
                                 int64_t batch, int64_t hq, int64_t hkv, int64_t d, int64_t capacity,
                                 const int32_t *lens, const int32_t *pos, int64_t max_len, int64_t max_pos,
                                 const attn_headprep_t *prep, double scale, int64_t splits,
                                 attn_dtype_t dtype, void *stream);

/*
 * Quantised KV cache (compute guide "Tensors, GPU kernels and AI models", Step 5: Run a
 * language model: keys and values kept in 8, 4 or 2 bits, or keys in 4 and values in 2,
 * each head coded over the range that returns it with the least squared error).
 *
 * Format of one cached tensor (K or V) with `bits` in {8, 4, 2}, head-major:
 *   codes  uint8 [batch, heads, capacity, d * bits / 8]: the d codes c of one head of one
 *          token; each 32-bit little-endian word holds 32 / bits consecutive codes, code
 *          j of the word at bit (j mod 2) * 16 + (j / 2) * bits (even codes in the low
 *          half-word, odd codes in the high half-word).
 *   params f32 [batch, heads, capacity, 2]: (lo, step); the head's value e is
 *          lo + step * c[e].
 * Coding (attn_kv_quantize): with L = 2^bits levels, min and max of the head's d values,
 * centre = (min + max) / 2, r = (max - min) / 2, candidate k = 0..23 has
 *   lo = centre - r (32 - k) / 32,  step = 2 r (32 - k) / 32 / (L - 1),
 *   c = clamp(rint((x - lo) * (1 / step)), 0, L - 1)       (f32, round to nearest even);
 * the candidate whose values lo + step c have the least squared error wins (the widest
 * on a tie; the error is summed in f64, so candidates within rounding of each other may
 * be ranked either way).  A head with r <= 1e-30 is coded lo = min, step = 0, c = 0.
 */

/*
 * attn_kv_quantize -- code rows of keys or values into a quantised cache.
 *   x       [batch, seq, heads, d] (row stride x_row_stride elements, sequences
 *           seq * x_row_stride apart), dtype ATTN_BF16 or ATTN_F32; read only.
 *   bits    8, 4 or 2.
 *   codes, params  the cache in the format above, with `capacity` rows per (sequence,
 *           head); token t of sequence b is written at row row0 + t.  16-byte aligned.
 *   0 <= row0, row0 + seq <= capacity.  d in {64, 128}.  batch or seq 0 is a no-op.
 * Keys are coded after their HeadPrep (run attn_prep on them first).
 */
attn_status_t attn_kv_quantize(const void *x, int64_t batch, int64_t seq, int64_t heads, int64_t d,
                               int64_t x_row_stride, int64_t bits, uint8_t *codes, float *params,
                               int64_t capacity, int64_t row0, attn_dtype_t dtype, void *stream);

/*
 * attn_decode_q -- attn_decode against a quantised cache: one new query row per
 * sequence attends the first lens[b] rows; the cache returns lo + step c per head.
 *   q, out       bf16 [batch, hq, d] contiguous (dtype must be ATTN_BF16).
 *   k_codes, k_params, v_codes, v_params   the caches (format above) with hkv heads and
 *                `capacity` rows, coded in k_bits and v_bits: (8, 8), (4, 4), (4, 2) or
 *                (2, 2).
 *   lens, pos, max_len, max_pos, prep, scale: as attn_decode.
 *   splits       number of key splits per sequence; 0 = attn_decode_q_default_splits
 *                (about one round of blocks: two per CU with 8-bit keys, three with 4- or
 *                2-bit keys, whose kernels hold fewer registers; at least 256 keys a split).
 *   workspace    at least attn_decode_workspace_size(batch, hq, hkv, d, max_len, s) bytes
 *                where s is the split count the call uses (the default resolved above
 *                when splits = 0); NULL is allowed when that size is 0.
 *   The products run on the matrix cores over the codes as bf16 operands, q carried as
 *   a bf16 high part plus a remainder; the errors are those of attn_decode's bf16 path.
 */
int64_t attn_decode_q_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t max_len,
                                     int64_t k_bits);
attn_status_t attn_decode_q(const void *q, const uint8_t *k_codes, const float *k_params,
                            const uint8_t *v_codes, const float *v_params, void *out, int64_t batch,
                            int64_t hq, int64_t hkv, int64_t d, int64_t capacity, int64_t k_bits,
                            int64_t v_bits, const int32_t *lens, const int32_t *pos, int64_t max_len,
                            int64_t max_pos, const attn_headprep_t *prep, double scale, int64_t splits, void *workspace,
                            size_t workspace_bytes, attn_dtype_t dtype, void *stream);

/*
 * attn_decode_q_paged -- attn_decode_q over a paged pool of coded rows.  Each page is a
 * quantised cache of batch 1 and capacity page_rows (codes [num_pages, hkv, page_rows,
 * d bits / 8], params [num_pages, hkv, page_rows, 2]), so attn_kv_quantize with
 * batch 1, capacity page_rows and row0 = the row in the page codes rows into a page.
 * pages, page_rows, num_pages, max_pages and the bad-page rule are attn_decode_paged's.
 */
attn_status_t attn_decode_q_paged(const void *q, const uint8_t *k_codes, const float *k_params,
                                  const uint8_t *v_codes, const float *v_params, void *out,
                                  int64_t batch, int64_t hq, int64_t hkv, int64_t d, int64_t num_pages,
                                  int64_t page_rows, int64_t k_bits, int64_t v_bits,
                                  const int32_t *pages, int64_t max_pages, const int32_t *lens,
                                  const int32_t *pos, int64_t max_len, int64_t max_pos,
                                  const attn_headprep_t *prep, double scale, int64_t splits,
                                  void *workspace, size_t workspace_bytes,
                                  attn_dtype_t dtype, void *stream);

/*
 * attn_rows -- full attention of packed rows, for image and video models (gizml:netops,
 * Functions > attentionRows, its BF16 path, and attendedRows for `queries`).
 *   qkv      [n, 3 * heads * head]: row r holds q, k and v of `heads` heads of `head`
 *            values each, in that order; contiguous.  With prep, the q heads of the
 *            query rows and the k heads of every row are prepped IN PLACE first (row r
 *            at table row r; prep->pairs selects split halves or adjacent pairs), so
 *            qkv changes; v is never written.
 *   group    0: every query sees every row's key.  > 0: the rows form groups of
 *            `group` consecutive rows (the last may be shorter) and a query sees only
 *            the keys of its own group (a block-diagonal mask).
 *   queries  0: every row is a query and out has n rows.  1 .. n: only the first
 *            `queries` rows are queries (each still sees the keys of its group, which
 *            may reach past row queries - 1) and out has `queries` rows.
 *   out      [queries or n, heads * head] contiguous; must not overlap qkv.
 *   The scale is 1 / sqrt(head); nothing is masked inside a group (no causal mask).
 *   head in {64, 128} (else ATTN_ERR_UNSUPPORTED); prep->table_rows >= n.  n == 0 is
 *   a no-op.  Up to three launches are enqueued (prep, the groups wholly made of
 *   queries, and the group holding the last queries).
 */
attn_status_t attn_rows(void *qkv, int64_t n, int64_t heads, int64_t head, int64_t group,
                        int64_t queries, void *out, const attn_headprep_t *prep,
                        attn_dtype_t dtype, void *stream);

/*
 * attn_rows8 -- attn_rows' quantised path (gizml:netops, Functions > attentionRows with
 * `quantized`: Q K^T on INT8, P V on E4M3 -- SageAttention's split -- with the head norm and
 * rotary applied in the quantizing pass; qkv is not written).  Same qkv, n, heads, head,
 * group, queries, out and prep as attn_rows (bf16 only, head in {64, 128}; prep: split
 * halves with half = head / 2 or 0, or adjacent pairs with any half); then:
 *   1. the quantizing pass writes the 8-bit operands into `workspace`:
 *        q8   int8 [nq, heads, head]   q after HeadPrep, one scale per (row, head):
 *        sq   f32  [nq, heads]         s = amax / 127, code = rint(x * (1 / s)) in [-127, 127]
 *        k8   int8 [n, heads, head]    k after HeadPrep, one scale per (tile, head), a tile
 *        sk   f32  [G, T, heads]       being 64 consecutive keys of a group (T tiles a group)
 *        v8t  E4M3 [G, T, heads, head, 64]  v over one scale per (group, head), s = amax /
 *        sv   f32  [G, heads]          448, nearest E4M3 of x * (1 / s), ties to even; row e
 *                                      of a tile's block holds value e of the tile's keys,
 *                                      position 32 g + b holding key
 *                                      32 (b / 16) + 8 ((b % 16) / 4) + 4 g + b % 4 (g < 2,
 *                                      b < 32); keys past the group's end are 0
 *        vmax f32  [G, T, heads]       scratch (each tile's amax of v)
 *      (G groups, nq = queries or n; an amax of 0 gives s = 1);
 *   2. out = softmax(q k^T / sqrt(head)) v over the values these give back, the weights
 *      carried as E4M3 numbers 2^(s - m) 448 with the running max m.
 * attn_rows8_layout fills offsets[0..6] with the byte offsets of q8, sq, k8, sk, v8t, sv,
 * vmax (256-byte aligned) and returns the workspace size (0 for bad sizes).
 * attn_rows8_quantize runs step 1 only, attn_rows8_attend step 2 only (on operands already
 * in the workspace), attn_rows8 both.  workspace: device memory of at least the layout's
 * size, 16-byte aligned, not overlapping qkv or out; calls sharing it must not overlap.
 */
size_t attn_rows8_layout(int64_t n, int64_t heads, int64_t head, int64_t group, int64_t queries,
                         int64_t *offsets);
attn_status_t attn_rows8_quantize(const void *qkv, int64_t n, int64_t heads, int64_t head,
                                  int64_t group, int64_t queries, const attn_headprep_t *prep,
                                  void *workspace, size_t workspace_bytes, void *stream);
attn_status_t attn_rows8_attend(const void *workspace, size_t workspace_bytes, int64_t n,
                                int64_t heads, int64_t head, int64_t group, int64_t queries,
                                void *out, void *stream);
attn_status_t attn_rows8(const void *qkv, int64_t n, int64_t heads, int64_t head, int64_t group,
                         int64_t queries, void *out, const attn_headprep_t *prep, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * attn_row_norm_rope -- a norm over the whole row followed by a per-head rotary, in
 * place (gizml:netops, Functions > rowNormRopeInto: LTX's QK norm, which spans every
 * head of a row, then its rotary).  For each row r of x:
 *   x[r, :] = x[r, :] / sqrt(mean over the width of x[r, :]^2 + eps) * w,
 *   then, if cos is given, each head h of `head` values turned by split halves: value
 *   d < head / 2 (a) with value d + head / 2 (b) as a' = a c - b s, b' = b c + a s,
 *   c = cos[r, h * head / 2 + d], s = sin[r, h * head / 2 + d].
 *   x          [rows, width] with rows row_stride elements apart; 16-byte aligned.
 *   width      8 <= width <= 8192, a multiple of 8.
 *   head       a multiple of 8 that divides width.
 *   row_stride >= width, a multiple of 8.
 *   w          device f32 [width], 16-byte aligned.
 *   cos, sin   device f32 [rows, width / 2] (row r serves row r of x), 16-byte aligned;
 *              both NULL: the norm only.
 *   eps        finite and >= 0 (taken as f32).
 *   dtype      storage type of x (the page's kernel is BF16; f32 is offered for exact
 *              checks); arithmetic is f32, rounded once to the storage type.
 *   rows == 0 is a no-op.  Errors: ATTN_ERR_ARG for the conditions above or
 *   rows >= 2^24; ATTN_ERR_UNSUPPORTED for an unknown dtype.
 */
attn_status_t attn_row_norm_rope(void *x, int64_t rows, int64_t width, int64_t head,
                                 int64_t row_stride, const float *w, const float *cos,
                                 const float *sin, double eps, attn_dtype_t dtype, void *stream);

/* 1 if head dim d and dtype are built into this library, else 0 (asked before
 * allocating, like gpukit's gkd_attention_ok). */
int attn_supported(int64_t d, attn_dtype_t dtype);

/* Static text for a status code. */
const char *attn_status_str(attn_status_t status);

/* Message of the last failed call on this thread ("" if none); valid until the
 * thread's next call into the library. */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
