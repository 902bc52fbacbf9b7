// kernels.h -- host-side launchers of the HIP kernels (internal to libattn).
//
// The C ABI layer (attn_api.cpp) validates every argument and then calls these.
// They only configure and enqueue launches; each returns the hipError_t of the
// enqueue.  Strides are in elements.
#pragma once

#include "common.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// HeadPrep of the tokens [0, seq) of `batch` sequences, for q and/or k.  src and dst
// may be the same buffer (in place).  Token t uses table row pos0 + t.  Token t of
// sequence b sits at b * bs + t * rs (elements); a batch stride of 0 means seq * rs.
struct PrepLaunch {
    const void *q_src; void *q_dst; int64_t q_src_rs, q_dst_rs; int64_t hq;
    const void *k_src; void *k_dst; int64_t k_src_rs, k_dst_rs; int64_t hkv;
    int64_t q_src_bs, q_dst_bs, k_src_bs, k_dst_bs;
    int64_t batch, seq, d, pos0;
    const float *qw, *kw, *cos, *sin;
    int64_t half;
    bool pairs;                  // turn adjacent pairs (2i, 2i + 1) rather than split halves
    float eps;
    bool bf16;
    // k_pages != NULL: k_dst is a paged pool and key row t of sequence b goes to pool row
    // pool_row(k_pages, b, k_row0 + t) (rows k_dst_rs apart); a row whose page id lies
    // outside the pool is not written.
    PageMap k_pages;
    int64_t k_row0;
    // past != NULL (device int32 [batch]): sequence b's rows sit at positions past[b] + t
    // (its table row, and its key's cache or pool row, k_dst not offset by the host);
    // past[b] outside [0, past_max] leaves sequence b's key rows unwritten.
    const int32_t *past;
    int64_t past_max;
};
hipError_t launch_prep(const PrepLaunch &a, hipStream_t stream);

// Attention of `seq` query rows per sequence against `tk` key rows (tk >= seq; 0 means
// tk = seq).  Query row i sits at position tk - seq + i (bottom-right alignment): with
// causal, it sees keys j <= i + tk - seq.  When prep_q is set, q's HeadPrep is applied
// as the q rows are read, query row i at table row pos0 + i (k must already be
// prepped).  Row t of sequence b sits at b * bs + t * rs (elements); a batch stride of
// 0 means rows * rs.
struct PrefillLaunch {
    const void *q; const void *k; const void *v; void *out;
    int64_t q_rs, k_rs, v_rs, o_rs;
    int64_t q_bs, k_bs, v_bs, o_bs;
    int64_t batch, seq, tk, hq, hkv, d, pos0;
    bool prep_q;                 // apply HeadPrep to q in the prologue
    const float *qw, *cos, *sin;
    const float *kwb;            // non-NULL: k was prepped with these weights (bounds |k|)
    float kmax;                  // > 0: caller's bound on every key row's norm
    PageMap kv_pages;            // pages != NULL: k, v are paged pools (rows k_rs / v_rs apart);
                                 // key j of sequence b is pool row pool_row(kv_pages, b, j)
    int64_t half;
    float eps;
    bool causal;
    float scale;
    bool bf16;
    // past != NULL (device int32 [batch], chunk mode): sequence b's query rows sit at
    // positions past[b] + i over its keys 0 .. past[b] + seq - 1; pos0 (= tk - seq) is
    // the host bound on every past[b], and one outside [0, pos0] gives NaN rows.
    const int32_t *past;
};
hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t stream);
// true if the fused q prologue of the chosen kernel can turn pairs `half` apart.
bool prefill_fuses_half(int64_t d, int64_t half, bool bf16);
// Fill the zero batch strides and tk of a prefill launch with their defaults.
void prefill_defaults(PrefillLaunch &a);

// Whole-row RMS norm (eps) times w [width], then with cos/sin [rows, width / 2] each
// head of `head` values turned by split halves at table entry h * head / 2 + d of its
// row; in place on `rows` rows `rs` elements apart.  width % 8 == 0, width <= 8192,
// head % 8 == 0 and divides width (checked by the caller).
struct RowNormRopeLaunch {
    void *x;
    int64_t rows, width, head, rs;
    const float *w, *cos, *sin;  // cos == NULL: norm only
    float eps;
    bool bf16;
};
hipError_t launch_row_norm_rope(const RowNormRopeLaunch &a, hipStream_t stream);

// Copy `rows` rows of `row_elems` elements of `batch` sequences (16-byte multiples,
// 16-byte aligned): row t of sequence b from src + b * src_bs + t * src_rs to
// dst + b * dst_bs + t * dst_rs (strides in elements of `elem` bytes).
struct CopyRowsLaunch {
    const void *src; void *dst;
    int64_t src_bs, src_rs, dst_bs, dst_rs;
    int64_t batch, rows, row_elems, elem;
    PageMap dst_pages;           // pages != NULL: row t of sequence b goes to pool row
    int64_t dst_row0;            // pool_row(dst_pages, b, dst_row0 + t); bad ids: not written
    // past != NULL: row t of sequence b goes to its row past[b] + t (dst not offset by
    // the host); past[b] outside [0, past_max]: not written.
    const int32_t *past;
    int64_t past_max;
};
hipError_t launch_copy_rows(const CopyRowsLaunch &a, hipStream_t stream);

struct DecodeLaunch {
    const void *q; const void *k; const void *v; void *out;
    int64_t batch, hq, hkv, d, capacity, max_len;
    const int32_t *lens, *pos;
    bool prep_q;
    const float *qw, *cos, *sin;
    int64_t half, table_rows;
    bool pairs;                  // turn adjacent pairs (2i, 2i + 1) rather than split halves
    float eps;
    float scale;
    int64_t splits;
    float *work;                 // [splits][batch][hq] x (d + 2) f32 partials
    bool bf16;
    // Quantised caches (kbits != 0): k and v hold codes [batch, hkv, capacity, d bits / 8]
    // (kbits for k, vbits for v, in {8, 4, 2}), kpar / vpar the (lo, step) f32 pairs
    // [batch, hkv, capacity, 2]; q and out are then bf16.
    const float *kpar, *vpar;
    int kbits, vbits;
    // Paged pool (pages != NULL): k and v hold num_pages pages of page_rows rows (a power
    // of two >= 16), each laid out as a cache of batch 1 and capacity page_rows; key j of
    // sequence b is row j % page_rows of page pages[b max_pages + j / page_rows].
    const int32_t *pages;
    int64_t page_rows, max_pages, num_pages;
};
hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream);
hipError_t launch_decode_q(const DecodeLaunch &a, hipStream_t stream);

// attentionRows' quantised path over packed rows qkv [n, 3 heads d] (bf16): groups of
// `group` rows (the last may be shorter), `tiles` 64-key tiles and `qtiles` 128-row query
// tiles per group; the first nq rows are queries.  The quantizing pass writes q8 [nq, heads,
// d] + sq [nq, heads], k8 [n, heads, d] + sk [groups, tiles, heads], v8t [groups, tiles,
// heads, d, 64] (E4M3, keys of a tile in the order the P V product takes them) + sv [groups,
// heads], using vmax [groups, tiles, heads] (each tile's amax of v) as scratch; the attention reads them and writes out
// [nq, heads d] (bf16).  prep_mode: 0 none, 1 split halves with half = d / 2, 2 pairs.
struct Rows8Launch {
    const void *qkv;
    int64_t n, nq, heads, d, group, groups, tiles, qtiles;
    const float *qw, *kw, *cos, *sin;
    int half, prep_mode;
    float eps;
    int8_t *q8; float *sq; int8_t *k8; float *sk; uint8_t *v8t; float *sv; float *vmax;
    void *out;
    float scale;
};
hipError_t launch_rows8_quantize(const Rows8Launch &a, hipStream_t stream);
hipError_t launch_rows8_attend(const Rows8Launch &a, hipStream_t stream);

// Quantised-cache coding of rows [0, seq) of `batch` sequences x [batch, seq, heads, d]
// (row stride rs, batch stride seq * rs elements) into cache rows row0 .. row0 + seq - 1:
// codes [batch, heads, capacity, d bits / 8], params [batch, heads, capacity, 2].
struct KvQuantLaunch {
    const void *x; int64_t rs;
    int64_t batch, seq, heads, d;
    int bits;
    uint8_t *codes; float *params;
    int64_t capacity, row0;
    bool bf16;
};
hipError_t launch_kv_quantize(const KvQuantLaunch &a, hipStream_t stream);

// Geometry of the decode split kernel, shared with the ABI layer's size queries.
int64_t decode_heads_per_block(int64_t hq, int64_t hkv);
// true when the bf16 decode runs as whole-row blocks (a wave per kv head)
bool decode_rows_fits(int64_t hq, int64_t hkv);
int64_t decode_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t d, int64_t max_len);
int64_t decode_q_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t max_len, int64_t kbits);
size_t decode_workspace_bytes(int64_t batch, int64_t hq, int64_t d, int64_t splits);
// The decode scratch that lives in the library (for callers that cannot allocate): its
// size, and its address on the current device (looked up once per device).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void **ptr);

}  // namespace attn
