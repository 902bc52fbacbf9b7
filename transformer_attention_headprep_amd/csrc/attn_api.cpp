// attn_api.cpp -- the C ABI of libattn: argument checks, then launches.
//
// Every entry point checks all of its arguments on the host before it enqueues
// anything, and returns an error code without touching the device when a check
// fails (the "validate and fail closed" convention of the gpukit page's devops
// wrappers).  Nothing here allocates or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/attn.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

attn_status_t fail(attn_status_t code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

attn_status_t hip_status(hipError_t err, const char *where) {
    if (err == hipSuccess) return ATTN_OK;
    return fail(ATTN_ERR_HIP, "%s: HIP error %d (%s)", where, (int)err, hipGetErrorString(err));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(attn_dtype_t dt) { return dt == ATTN_BF16 ? 2 : 4; }

attn_status_t check_dtype_d(attn_dtype_t dt, int64_t d) {
    if (dt != ATTN_F32 && dt != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim %lld not in {64, 128}", (long long)d);
    return ATTN_OK;
}

// A [batch, seq, heads, d] operand with row stride rs.
attn_status_t check_rows(const char *name, const void *p, int64_t heads, int64_t d, int64_t rs) {
    if (!p) return fail(ATTN_ERR_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(ATTN_ERR_ARG, "%s is not 16-byte aligned", name);
    if (heads <= 0) return fail(ATTN_ERR_ARG, "%s: head count %lld <= 0", name, (long long)heads);
    if (rs < heads * d) return fail(ATTN_ERR_ARG, "%s: row stride %lld < heads * d = %lld", name, (long long)rs, (long long)(heads * d));
    if (rs % 8 != 0) return fail(ATTN_ERR_ARG, "%s: row stride %lld not a multiple of 8 elements", name, (long long)rs);
    if (rs >= ((int64_t)1 << 24)) return fail(ATTN_ERR_ARG, "%s: row stride %lld >= 2^24 elements", name, (long long)rs);
    return ATTN_OK;
}

struct Span { uintptr_t lo, hi; };

Span span(const void *p, int64_t rows, int64_t rs, int64_t heads, int64_t d, size_t es) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    const uintptr_t hi = lo + (uintptr_t)(((rows - 1) * rs + heads * d) * (int64_t)es);
    return {lo, hi};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// The HeadPrep record: tables cover positions [first, first + count).
attn_status_t check_prep(const attn_headprep_t *p, int64_t d, bool need_qw, bool need_kw, int64_t first,
                         int64_t count) {
    if (need_qw && !p->qw) return fail(ATTN_ERR_ARG, "prep->qw is NULL");
    if (need_kw && !p->kw) return fail(ATTN_ERR_ARG, "prep->kw is NULL");
    if ((need_qw && !aligned16(p->qw)) || (need_kw && !aligned16(p->kw)))
        return fail(ATTN_ERR_ARG, "prep weights are not 16-byte aligned");
    if (!(p->eps >= 0.0) || !std::isfinite(p->eps)) return fail(ATTN_ERR_ARG, "prep->eps must be finite and >= 0");
    if (p->pairs != 0 && p->pairs != 1) return fail(ATTN_ERR_ARG, "prep->pairs = %lld not 0 or 1", (long long)p->pairs);
    if (!(p->kmax >= 0.0) || !std::isfinite(p->kmax) || p->kmax > 3.0e38)
        return fail(ATTN_ERR_ARG, "prep->kmax must be finite and >= 0");
    if (p->half < 0 || 2 * p->half > d)
        return fail(ATTN_ERR_ARG, "prep->half = %lld outside [0, d/2]", (long long)p->half);
    if (p->half > 0) {
        if (!p->cos || !p->sin) return fail(ATTN_ERR_ARG, "prep->cos/sin is NULL with half > 0");
        if (!aligned16(p->cos) || !aligned16(p->sin)) return fail(ATTN_ERR_ARG, "prep tables are not 16-byte aligned");
        if (p->table_rows <= 0) return fail(ATTN_ERR_ARG, "prep->table_rows <= 0");
        if (count > 0 && (first < 0 || first + count > p->table_rows))
            return fail(ATTN_ERR_ARG, "positions [%lld, %lld) outside the %lld-row table", (long long)first,
                        (long long)(first + count), (long long)p->table_rows);
    }
    return ATTN_OK;
}

// Geometry and workspace layout of the quantised rows path (see attn_rows8 in attn.h).
struct Rows8Geo {
    int64_t nq, G, groups, tiles, qtiles;
    int64_t off[7];
    size_t total;
};

bool rows8_geo(int64_t n, int64_t heads, int64_t head, int64_t group, int64_t queries, Rows8Geo &g) {
    if (n <= 0 || heads <= 0 || (head != 64 && head != 128) || group < 0 || queries < 0 || queries > n) return false;
    g.nq = queries ? queries : n;
    g.G = (group == 0 || group > n) ? n : group;
    g.groups = (n + g.G - 1) / g.G;
    g.tiles = (g.G + 63) / 64;
    g.qtiles = (g.G + 127) / 128;
    const int64_t sizes[7] = {g.nq * heads * head, g.nq * heads * 4, n * heads * head, g.groups * g.tiles * heads * 4,
                              g.groups * g.tiles * heads * head * 64, g.groups * heads * 4, g.groups * g.tiles * heads * 4};
    int64_t at = 0;
    for (int i = 0; i < 7; ++i) {
        g.off[i] = at;
        at += (sizes[i] + 255) / 256 * 256;
    }
    g.total = (size_t)at;
    return true;
}

attn_status_t rows8_launch(const void *qkv, int64_t n, int64_t heads, int64_t head, int64_t group, int64_t queries,
                           void *out, const attn_headprep_t *prep, const void *workspace, size_t workspace_bytes,
                           bool quantize, bool attend, void *stream) {
    attn_status_t st;
    if (n < 0) return fail(ATTN_ERR_ARG, "n < 0");
    if (head != 64 && head != 128) return fail(ATTN_ERR_UNSUPPORTED, "head %lld not in {64, 128}", (long long)head);
    if (heads <= 0) return fail(ATTN_ERR_ARG, "heads <= 0");
    if (group < 0) return fail(ATTN_ERR_ARG, "group < 0");
    if (queries < 0 || queries > n) return fail(ATTN_ERR_ARG, "queries %lld outside [0, n = %lld]", (long long)queries, (long long)n);
    const int64_t rs = 3 * heads * head;
    if (quantize && (st = check_rows("qkv", qkv, 3 * heads, head, rs))) return st;
    if (attend && (st = check_rows("out", out, heads, head, heads * head))) return st;
    int mode = 0;
    if (quantize && prep) {
        if ((st = check_prep(prep, head, true, true, 0, n))) return st;
        if (prep->half > 0) {
            if (prep->pairs) mode = 2;
            else if (2 * prep->half == head) mode = 1;
            else return fail(ATTN_ERR_UNSUPPORTED, "the quantised path turns split halves only with half = head / 2");
        } else {
            mode = 1;   // norm and weight only
        }
    }
    if (n == 0) return ATTN_OK;
    Rows8Geo geo;
    rows8_geo(n, heads, head, group, queries, geo);
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is NULL");
    if (workspace_bytes < geo.total)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, geo.total);
    if (!aligned16(workspace)) return fail(ATTN_ERR_ARG, "workspace is not 16-byte aligned");
    if (geo.groups * geo.tiles >= ((int64_t)1 << 31) || heads >= 65536 || n >= ((int64_t)1 << 31) ||
        (quantize && prep && n * prep->half * 4 >= ((int64_t)1 << 31)) || 64 * rs * 2 >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_ARG, "problem too large for one launch");
    const Span sw{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + geo.total};
    if (quantize && overlap(sw, span(qkv, n, rs, 3 * heads, head, 2))) return fail(ATTN_ERR_ARG, "workspace overlaps qkv");
    if (attend && overlap(sw, span(out, geo.nq, heads * head, heads, head, 2))) return fail(ATTN_ERR_ARG, "workspace overlaps out");
    if (quantize && attend && overlap(span(out, geo.nq, heads * head, heads, head, 2), span(qkv, n, rs, 3 * heads, head, 2)))
        return fail(ATTN_ERR_ARG, "out overlaps qkv");
    uint8_t *ws = static_cast<uint8_t *>(const_cast<void *>(workspace));
    attn::Rows8Launch a{};
    a.qkv = qkv; a.n = n; a.nq = geo.nq; a.heads = heads; a.d = head; a.group = geo.G; a.groups = geo.groups;
    a.tiles = geo.tiles; a.qtiles = geo.qtiles;
    a.prep_mode = mode;
    if (quantize && prep) {
        a.qw = prep->qw; a.kw = prep->kw; a.cos = prep->cos; a.sin = prep->sin;
        a.half = (int)prep->half; a.eps = (float)prep->eps;
    }
    a.q8 = reinterpret_cast<int8_t *>(ws + geo.off[0]); a.sq = reinterpret_cast<float *>(ws + geo.off[1]);
    a.k8 = reinterpret_cast<int8_t *>(ws + geo.off[2]); a.sk = reinterpret_cast<float *>(ws + geo.off[3]);
    a.v8t = ws + geo.off[4]; a.sv = reinterpret_cast<float *>(ws + geo.off[5]);
    a.vmax = reinterpret_cast<float *>(ws + geo.off[6]);
    a.out = out; a.scale = (float)(1.0 / std::sqrt((double)head));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (quantize && (st = hip_status(attn::launch_rows8_quantize(a, s), "attn_rows8 (quantize)"))) return st;
    if (attend && (st = hip_status(attn::launch_rows8_attend(a, s), "attn_rows8 (attend)"))) return st;
    return ATTN_OK;
}

// A paged KV pool: the page table and its sizes.
struct Paging {
    const int32_t *pages;      // [batch, max_pages] pool page of each sequence's rows
    int64_t page_rows, max_pages, num_pages;
};

attn_status_t check_paging(const Paging &pg, int64_t max_len, int64_t batch) {
    if (!pg.pages) return fail(ATTN_ERR_ARG, "pages is NULL");
    if ((reinterpret_cast<uintptr_t>(pg.pages) & 3) != 0) return fail(ATTN_ERR_ARG, "pages is not 4-byte aligned");
    if (pg.page_rows < 16 || pg.page_rows > ((int64_t)1 << 20) || (pg.page_rows & (pg.page_rows - 1)) != 0)
        return fail(ATTN_ERR_ARG, "page_rows %lld is not a power of two in [16, 2^20]", (long long)pg.page_rows);
    if (pg.num_pages < 1 || pg.num_pages * pg.page_rows >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_ARG, "num_pages %lld outside [1, 2^31 / page_rows)", (long long)pg.num_pages);
    if (pg.max_pages < 1 || batch * pg.max_pages >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_ARG, "max_pages %lld outside [1, 2^31 / batch)", (long long)pg.max_pages);
    if (max_len < 1 || max_len > pg.max_pages * pg.page_rows)
        return fail(ATTN_ERR_ARG, "max_len %lld outside [1, max_pages * page_rows]", (long long)max_len);
    return ATTN_OK;
}

Span table_span(const Paging &pg, int64_t batch) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(pg.pages);
    return Span{a, a + (uintptr_t)(batch * pg.max_pages * 4)};
}

}  // namespace

extern "C" {

size_t attn_rows8_layout(int64_t n, int64_t heads, int64_t head, int64_t group, int64_t queries, int64_t *offsets) {
    Rows8Geo geo;
    if (!rows8_geo(n, heads, head, group, queries, geo)) return 0;
    if (offsets)
        for (int i = 0; i < 7; ++i) offsets[i] = geo.off[i];
    return geo.total;
}

attn_status_t attn_rows8_quantize(const void *qkv, int64_t n, int64_t heads, int64_t head, int64_t group,
                                  int64_t queries, const attn_headprep_t *prep, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    g_last_error[0] = 0;
    return rows8_launch(qkv, n, heads, head, group, queries, nullptr, prep, workspace, workspace_bytes, true, false,
                        stream);
}

attn_status_t attn_rows8_attend(const void *workspace, size_t workspace_bytes, int64_t n, int64_t heads, int64_t head,
                                int64_t group, int64_t queries, void *out, void *stream) {
    g_last_error[0] = 0;
    return rows8_launch(nullptr, n, heads, head, group, queries, out, nullptr, workspace, workspace_bytes, false, true,
                        stream);
}

attn_status_t attn_rows8(const void *qkv, int64_t n, int64_t heads, int64_t head, int64_t group, int64_t queries,
                         void *out, const attn_headprep_t *prep, void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    return rows8_launch(qkv, n, heads, head, group, queries, out, prep, workspace, workspace_bytes, true, true, stream);
}

const char *attn_last_error(void) { return g_last_error; }

const char *attn_status_str(attn_status_t s) {
    switch (s) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_ARG: return "invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported head dim or dtype";
        case ATTN_ERR_WORKSPACE: return "workspace too small";
        case ATTN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int attn_supported(int64_t d, attn_dtype_t dt) {
    return (d == 64 || d == 128) && (dt == ATTN_F32 || dt == ATTN_BF16);
}

attn_status_t attn_prep(void *q, void *k, int64_t batch, int64_t seq, int64_t hq, int64_t hkv, int64_t d,
                        int64_t q_row_stride, int64_t k_row_stride, int64_t pos0, const attn_headprep_t *prep,
                        attn_dtype_t dtype, void *stream) {
    g_last_error[0] = 0;
    attn_status_t st = check_dtype_d(dtype, d);
    if (st) return st;
    if (!prep) return fail(ATTN_ERR_ARG, "prep is NULL");
    if (!q && !k) return fail(ATTN_ERR_ARG, "q and k are both NULL");
    if (batch < 0 || seq < 0) return fail(ATTN_ERR_ARG, "negative batch or seq");
    if (q && (st = check_rows("q", q, hq, d, q_row_stride))) return st;
    if (k && (st = check_rows("k", k, hkv, d, k_row_stride))) return st;
    if ((st = check_prep(prep, d, q != nullptr, k != nullptr, pos0, seq))) return st;
    if (pos0 < 0) return fail(ATTN_ERR_ARG, "pos0 < 0");
    if (batch == 0 || seq == 0) return ATTN_OK;
    const size_t es = elem_size(dtype);
    if (q && k && overlap(span(q, batch * seq, q_row_stride, hq, d, es), span(k, batch * seq, k_row_stride, hkv, d, es))) {
        // Packed qkv rows interleave q and k; they only clash if a q head lands on a k head.
        const intptr_t delta = reinterpret_cast<intptr_t>(k) - reinterpret_cast<intptr_t>(q);
        if (q_row_stride != k_row_stride || delta % (intptr_t)es != 0)
            return fail(ATTN_ERR_ARG, "q and k overlap");
        const int64_t off = delta / (intptr_t)es;
        if (!(off >= hq * d && off + hkv * d <= q_row_stride) && !(-off >= hkv * d && -off + hq * d <= q_row_stride))
            return fail(ATTN_ERR_ARG, "q and k overlap");
    }
    attn::PrepLaunch a{};
    a.q_src = q; a.q_dst = q; a.q_src_rs = q_row_stride; a.q_dst_rs = q_row_stride; a.hq = hq;
    a.k_src = k; a.k_dst = k; a.k_src_rs = k_row_stride; a.k_dst_rs = k_row_stride; a.hkv = hkv;
    a.batch = batch; a.seq = seq; a.d = d; a.pos0 = pos0;
    a.qw = prep->qw; a.kw = prep->kw; a.cos = prep->cos; a.sin = prep->sin;
    a.half = prep->half; a.pairs = prep->pairs != 0; a.eps = (float)prep->eps; a.bf16 = dtype == ATTN_BF16;
    return hip_status(attn::launch_prep(a, static_cast<hipStream_t>(stream)), "attn_prep");
}

attn_status_t attn_prefill(const void *q, void *k, const void *v, void *out, int64_t batch, int64_t seq, int64_t hq,
                           int64_t hkv, int64_t d, int64_t q_row_stride, int64_t k_row_stride,
                           int64_t v_row_stride, int64_t o_row_stride, int64_t pos0, const attn_headprep_t *prep,
                           int causal, double scale, attn_dtype_t dtype, void *stream) {
    g_last_error[0] = 0;
    attn_status_t st = check_dtype_d(dtype, d);
    if (st) return st;
    if (batch < 0 || seq < 0) return fail(ATTN_ERR_ARG, "negative batch or seq");
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
        return fail(ATTN_ERR_ARG, "hq = %lld must be a positive multiple of hkv = %lld", (long long)hq, (long long)hkv);
    if ((st = check_rows("q", q, hq, d, q_row_stride))) return st;
    if ((st = check_rows("k", k, hkv, d, k_row_stride))) return st;
    if ((st = check_rows("v", v, hkv, d, v_row_stride))) return st;
    if ((st = check_rows("out", out, hq, d, o_row_stride))) return st;
    if (!std::isfinite(scale) || !(scale > 0.0)) return fail(ATTN_ERR_ARG, "scale must be finite and > 0");
    if (prep) {
        if ((st = check_prep(prep, d, true, false, pos0, seq))) return st;
        if (pos0 < 0) return fail(ATTN_ERR_ARG, "pos0 < 0");
    }
    if (batch == 0 || seq == 0) return ATTN_OK;
    if ((int64_t)((seq + 127) / 128) * batch * hq >= (int64_t)1 << 31 || seq >= (int64_t)1 << 31)
        return fail(ATTN_ERR_ARG, "problem too large for one launch");
    const size_t es = elem_size(dtype);
    const int64_t rows = batch * seq;
    const Span so = span(out, rows, o_row_stride, hq, d, es);
    if (overlap(so, span(q, rows, q_row_stride, hq, d, es)) || overlap(so, span(k, rows, k_row_stride, hkv, d, es)) ||
        overlap(so, span(v, rows, v_row_stride, hkv, d, es)))
        return fail(ATTN_ERR_ARG, "out overlaps q, k or v");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = dtype == ATTN_BF16;

    attn::PrefillLaunch a{};
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.q_rs = q_row_stride; a.k_rs = k_row_stride; a.v_rs = v_row_stride; a.o_rs = o_row_stride;
    a.batch = batch; a.seq = seq; a.hq = hq; a.hkv = hkv; a.d = d; a.pos0 = pos0;
    a.causal = causal != 0; a.scale = (float)scale; a.bf16 = bf16;
    if (prep) {
        const bool fused = !prep->pairs && attn::prefill_fuses_half(d, prep->half, bf16);
        // k is prepped in place; q either in the attention prologue or, for halves the
        // prologue cannot turn, into `out` first (each attention block then reads its
        // q rows from out before it overwrites exactly those rows).
        // prep->kw == NULL: k already holds prepped keys and is left as it is.
        attn::PrepLaunch pa{};
        if (prep->kw) {
            pa.k_src = k; pa.k_dst = k; pa.k_src_rs = k_row_stride; pa.k_dst_rs = k_row_stride; pa.hkv = hkv;
        }
        if (!fused) {
            pa.q_src = q; pa.q_dst = out; pa.q_src_rs = q_row_stride; pa.q_dst_rs = o_row_stride; pa.hq = hq;
        }
        pa.batch = batch; pa.seq = seq; pa.d = d; pa.pos0 = pos0;
        pa.qw = prep->qw; pa.kw = prep->kw; pa.cos = prep->cos; pa.sin = prep->sin;
        pa.half = prep->half; pa.pairs = prep->pairs != 0; pa.eps = (float)prep->eps; pa.bf16 = bf16;
        if (pa.k_src || pa.q_src)
            if ((st = hip_status(attn::launch_prep(pa, s), "attn_prefill (prep)"))) return st;
        if (fused) {
            a.prep_q = true;
            a.qw = prep->qw; a.cos = prep->cos; a.sin = prep->sin; a.half = prep->half; a.eps = (float)prep->eps;
            a.kwb = prep->kw;            // k was prepped with kw just above
            a.kmax = (float)prep->kmax;
        } else {
            a.q = out; a.q_rs = o_row_stride;
        }
    }
    return hip_status(attn::launch_prefill(a, s), "attn_prefill");
}

static attn_status_t chunk_impl(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                void *out, int64_t batch, int64_t tq, int64_t hq, int64_t hkv, int64_t d,
                                int64_t capacity, const Paging *pg, int64_t n_past, const int32_t *past,
                                const attn_headprep_t *prep, int causal, double scale, attn_dtype_t dtype,
                                void *stream) {
    g_last_error[0] = 0;
    attn_status_t st = check_dtype_d(dtype, d);
    if (st) return st;
    if (pg && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "paged pools hold bf16 rows");
    if (batch < 0 || tq < 0) return fail(ATTN_ERR_ARG, "negative batch or tq");
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
        return fail(ATTN_ERR_ARG, "hq = %lld must be a positive multiple of hkv = %lld", (long long)hq, (long long)hkv);
    if ((st = check_rows("q", q, hq, d, hq * d))) return st;
    if ((st = check_rows("k_new", k_new, hkv, d, hkv * d))) return st;
    if ((st = check_rows("v_new", v_new, hkv, d, hkv * d))) return st;
    if ((st = check_rows("k_cache", k_cache, hkv, d, hkv * d))) return st;
    if ((st = check_rows("v_cache", v_cache, hkv, d, hkv * d))) return st;
    if ((st = check_rows("out", out, hq, d, hq * d))) return st;
    int64_t cache_rows;                        // rows the cache pointers span
    if (pg) {
        if (pg->page_rows < 64) return fail(ATTN_ERR_ARG, "page_rows %lld < 64", (long long)pg->page_rows);
        if (n_past < 0) return fail(ATTN_ERR_ARG, "n_past < 0");
        if ((st = check_paging(*pg, std::max<int64_t>(n_past + tq, 1), batch))) return st;
        cache_rows = pg->num_pages * pg->page_rows;
    } else {
        if (capacity <= 0 || capacity >= ((int64_t)1 << 31)) return fail(ATTN_ERR_ARG, "capacity %lld outside [1, 2^31)", (long long)capacity);
        if (n_past < 0 || n_past + tq > capacity)
            return fail(ATTN_ERR_ARG, "n_past %lld + tq %lld outside [0, capacity %lld]", (long long)n_past, (long long)tq,
                        (long long)capacity);
        cache_rows = batch * capacity;
    }
    if (!std::isfinite(scale) || !(scale > 0.0)) return fail(ATTN_ERR_ARG, "scale must be finite and > 0");
    const bool prep_k = prep && prep->kw;
    if (prep && (st = check_prep(prep, d, true, false, n_past, tq))) return st;
    if (prep_k && !aligned16(prep->kw)) return fail(ATTN_ERR_ARG, "prep weights are not 16-byte aligned");
    if (batch == 0 || tq == 0) return ATTN_OK;
    if ((int64_t)((tq + 127) / 128) * batch * hq >= (int64_t)1 << 31)
        return fail(ATTN_ERR_ARG, "problem too large for one launch");
    const size_t es = elem_size(dtype);
    const Span so = span(out, batch * tq, hq * d, hq, d, es);
    const Span sq = span(q, batch * tq, hq * d, hq, d, es);
    const Span skn = span(k_new, batch * tq, hkv * d, hkv, d, es);
    const Span svn = span(v_new, batch * tq, hkv * d, hkv, d, es);
    const Span skc = span(k_cache, cache_rows, hkv * d, hkv, d, es);
    const Span svc = span(v_cache, cache_rows, hkv * d, hkv, d, es);
    if (overlap(so, sq) || overlap(so, skn) || overlap(so, svn) || overlap(so, skc) || overlap(so, svc) ||
        (pg && overlap(so, table_span(*pg, batch))))
        return fail(ATTN_ERR_ARG, "out overlaps another buffer");
    if (pg && (overlap(skc, table_span(*pg, batch)) || overlap(svc, table_span(*pg, batch))))
        return fail(ATTN_ERR_ARG, "the page table overlaps a pool");
    if (overlap(skc, svc) || overlap(skn, skc) || overlap(skn, svc) || overlap(svn, skc) || overlap(svn, svc))
        return fail(ATTN_ERR_ARG, "the caches overlap each other or the new rows");
    if (past) {
        const Span sp{reinterpret_cast<uintptr_t>(past), reinterpret_cast<uintptr_t>(past + batch)};
        if (overlap(sp, so) || overlap(sp, skc) || overlap(sp, svc))
            return fail(ATTN_ERR_ARG, "past overlaps out or a cache");
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = dtype == ATTN_BF16;
    const int64_t crs = hkv * d, cbs = pg ? 0 : capacity * crs;    // cache row and sequence strides
    attn::PageMap pm{};
    if (pg) {
        pm.pages = pg->pages; pm.max_pages = (int)pg->max_pages; pm.num_pages = (int)pg->num_pages;
        while (((int64_t)1 << pm.shift) < pg->page_rows) ++pm.shift;
    }

    // 1-2. Append: prepped keys and values into cache rows n_past .. n_past + tq - 1 (of
    // each sequence's pages, with a pool); with per-sequence lengths, rows past[b] .. of
    // sequence b (the kernels offset each sequence themselves).
    const int64_t host_row0 = past ? 0 : n_past;
    attn::CopyRowsLaunch cv{};
    cv.src = v_new;
    cv.dst = pg ? v_cache : static_cast<uint8_t *>(v_cache) + (size_t)(host_row0 * crs) * es;
    cv.src_bs = tq * crs; cv.src_rs = crs; cv.dst_bs = cbs; cv.dst_rs = crs;
    cv.batch = batch; cv.rows = tq; cv.row_elems = crs; cv.elem = (int64_t)es;
    cv.dst_pages = pm; cv.dst_row0 = host_row0;
    cv.past = past; cv.past_max = n_past;
    void *k_dst = pg ? k_cache : static_cast<uint8_t *>(k_cache) + (size_t)(host_row0 * crs) * es;
    if (prep_k) {
        attn::PrepLaunch pk{};
        pk.k_src = k_new; pk.k_dst = k_dst; pk.k_src_rs = crs; pk.k_dst_rs = crs; pk.hkv = hkv;
        pk.k_src_bs = tq * crs; pk.k_dst_bs = cbs;              // (unused with a pool)
        pk.k_pages = pm; pk.k_row0 = host_row0;
        pk.past = past; pk.past_max = n_past;
        pk.batch = batch; pk.seq = tq; pk.d = d; pk.pos0 = n_past;
        pk.qw = prep->qw; pk.kw = prep->kw; pk.cos = prep->cos; pk.sin = prep->sin;
        pk.half = prep->half; pk.pairs = prep->pairs != 0; pk.eps = (float)prep->eps; pk.bf16 = bf16;
        if ((st = hip_status(attn::launch_prep(pk, s), "attn_prefill_chunk (k prep)"))) return st;
    } else {
        attn::CopyRowsLaunch ck = cv;
        ck.src = k_new; ck.dst = k_dst;
        if ((st = hip_status(attn::launch_copy_rows(ck, s), "attn_prefill_chunk (k copy)"))) return st;
    }
    if ((st = hip_status(attn::launch_copy_rows(cv, s), "attn_prefill_chunk (v copy)"))) return st;

    // 3. Attention of the chunk's queries over cache rows 0 .. n_past + tq - 1.
    attn::PrefillLaunch a{};
    a.q = q; a.k = k_cache; a.v = v_cache; a.out = out;
    a.q_rs = hq * d; a.k_rs = crs; a.v_rs = crs; a.o_rs = hq * d;
    a.k_bs = cbs; a.v_bs = cbs;                       // (unused with a pool)
    a.kv_pages = pm;
    a.batch = batch; a.seq = tq; a.tk = n_past + tq; a.hq = hq; a.hkv = hkv; a.d = d; a.pos0 = n_past;
    a.causal = causal != 0; a.scale = (float)scale; a.bf16 = bf16;
    a.past = past;
    if (prep) {
        if (!prep->pairs && attn::prefill_fuses_half(d, prep->half, bf16)) {
            a.prep_q = true;
            a.qw = prep->qw; a.cos = prep->cos; a.sin = prep->sin; a.half = prep->half; a.eps = (float)prep->eps;
            a.kmax = (float)prep->kmax;  // cached rows: only the caller's bound
        } else {
            // q prepped into out first; each attention block reads exactly the rows it writes.
            attn::PrepLaunch pq{};
            pq.q_src = q; pq.q_dst = out; pq.q_src_rs = hq * d; pq.q_dst_rs = hq * d; pq.hq = hq;
            pq.batch = batch; pq.seq = tq; pq.d = d; pq.pos0 = n_past;
            pq.past = past; pq.past_max = n_past;
            pq.qw = prep->qw; pq.cos = prep->cos; pq.sin = prep->sin;
            pq.half = prep->half; pq.pairs = prep->pairs != 0; pq.eps = (float)prep->eps; pq.bf16 = bf16;
            if ((st = hip_status(attn::launch_prep(pq, s), "attn_prefill_chunk (q prep)"))) return st;
            a.q = out;
        }
    }
    return hip_status(attn::launch_prefill(a, s), pg ? "attn_prefill_chunk_paged" : "attn_prefill_chunk");
}

attn_status_t attn_prefill_chunk(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                 void *out, int64_t batch, int64_t tq, int64_t hq, int64_t hkv, int64_t d,
                                 int64_t capacity, int64_t n_past, const int32_t *past,
                                 const attn_headprep_t *prep, int causal, double scale, attn_dtype_t dtype,
                                 void *stream) {
    return chunk_impl(q, k_new, v_new, k_cache, v_cache, out, batch, tq, hq, hkv, d, capacity, nullptr, n_past, past,
                      prep, causal, scale, dtype, stream);
}

attn_status_t attn_prefill_chunk_paged(const void *q, const void *k_new, const void *v_new, void *k_pool,
                                       void *v_pool, void *out, int64_t batch, int64_t tq, int64_t hq, int64_t hkv,
                                       int64_t d, int64_t num_pages, int64_t page_rows, const int32_t *pages,
                                       int64_t max_pages, int64_t n_past, const int32_t *past,
                                       const attn_headprep_t *prep, int causal, double scale, attn_dtype_t dtype,
                                       void *stream) {
    const Paging pg{pages, page_rows, max_pages, num_pages};
    return chunk_impl(q, k_new, v_new, k_pool, v_pool, out, batch, tq, hq, hkv, d, 0, &pg, n_past, past, prep, causal,
                      scale, dtype, stream);
}

attn_status_t attn_rows(void *qkv, int64_t n, int64_t heads, int64_t head, int64_t group, int64_t queries, void *out,
                        const attn_headprep_t *prep, attn_dtype_t dtype, void *stream) {
    g_last_error[0] = 0;
    attn_status_t st = check_dtype_d(dtype, head);
    if (st) return st;
    if (n < 0) return fail(ATTN_ERR_ARG, "n < 0");
    if (heads <= 0) return fail(ATTN_ERR_ARG, "heads <= 0");
    const int64_t rs = 3 * heads * head, ors = heads * head;
    if ((st = check_rows("qkv", qkv, 3 * heads, head, rs))) return st;
    if ((st = check_rows("out", out, heads, head, ors))) return st;
    if (group < 0) return fail(ATTN_ERR_ARG, "group < 0");
    if (queries < 0 || queries > n) return fail(ATTN_ERR_ARG, "queries %lld outside [0, n = %lld]", (long long)queries, (long long)n);
    if (prep && (st = check_prep(prep, head, true, true, 0, n))) return st;
    if (n == 0) return ATTN_OK;
    const int64_t nq = queries ? queries : n;
    const int64_t G = (group == 0 || group > n) ? n : group;
    if (n >= ((int64_t)1 << 31) || ((G + 127) / 128) * ((nq + G - 1) / G) * heads >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_ARG, "problem too large for one launch");
    const size_t es = elem_size(dtype);
    if (overlap(span(out, nq, ors, heads, head, es), span(qkv, n, rs, 3 * heads, head, es)))
        return fail(ATTN_ERR_ARG, "out overlaps qkv");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = dtype == ATTN_BF16;
    uint8_t *base = static_cast<uint8_t *>(qkv);
    void *qp = base, *kp = base + (size_t)(heads * head) * es, *vp = base + (size_t)(2 * heads * head) * es;

    // HeadPrep in place first: q of the query rows, k of every row, row r at table row r.
    if (prep) {
        attn::PrepLaunch pa{};
        pa.k_src = kp; pa.k_dst = kp; pa.k_src_rs = rs; pa.k_dst_rs = rs; pa.hkv = heads;
        pa.batch = 1; pa.seq = n; pa.d = head; pa.pos0 = 0;
        pa.qw = prep->qw; pa.kw = prep->kw; pa.cos = prep->cos; pa.sin = prep->sin;
        pa.half = prep->half; pa.pairs = prep->pairs != 0; pa.eps = (float)prep->eps; pa.bf16 = bf16;
        attn::PrepLaunch pq = pa;
        pq.k_src = nullptr; pq.k_dst = nullptr;
        pq.q_src = qp; pq.q_dst = qp; pq.q_src_rs = rs; pq.q_dst_rs = rs; pq.hq = heads; pq.seq = nq;
        if (nq == n) {   // one launch for both
            pa.q_src = qp; pa.q_dst = qp; pa.q_src_rs = rs; pa.q_dst_rs = rs; pa.hq = heads;
        } else if ((st = hip_status(attn::launch_prep(pq, s), "attn_rows (q prep)"))) {
            return st;
        }
        if ((st = hip_status(attn::launch_prep(pa, s), "attn_rows (prep)"))) return st;
    }

    // Full attention inside each group of G rows: the groups whose rows are all queries
    // form one batched launch; the queries left over (the start of the next group) attend
    // that group's keys in a second one.
    attn::PrefillLaunch a{};
    a.q_rs = rs; a.k_rs = rs; a.v_rs = rs; a.o_rs = ors;
    a.hq = heads; a.hkv = heads; a.d = head; a.causal = false; a.bf16 = bf16;
    a.scale = (float)(1.0 / std::sqrt((double)head));
    const int64_t full = nq / G;
    if (full > 0) {
        attn::PrefillLaunch f = a;
        f.q = qp; f.k = kp; f.v = vp; f.out = out;
        f.q_bs = G * rs; f.k_bs = G * rs; f.v_bs = G * rs; f.o_bs = G * ors;
        f.batch = full; f.seq = G; f.tk = G;
        if ((st = hip_status(attn::launch_prefill(f, s), "attn_rows"))) return st;
    }
    const int64_t r0 = full * G, tq = nq - r0;
    if (tq > 0) {
        attn::PrefillLaunch t = a;
        const size_t off = (size_t)(r0 * rs) * es;
        t.q = base + off; t.k = static_cast<uint8_t *>(kp) + off; t.v = static_cast<uint8_t *>(vp) + off;
        t.out = static_cast<uint8_t *>(out) + (size_t)(r0 * ors) * es;
        t.batch = 1; t.seq = tq; t.tk = std::min(G, n - r0);
        if ((st = hip_status(attn::launch_prefill(t, s), "attn_rows (tail)"))) return st;
    }
    return ATTN_OK;
}

attn_status_t attn_row_norm_rope(void *x, int64_t rows, int64_t width, int64_t head, int64_t row_stride,
                                 const float *w, const float *cos, const float *sin, double eps, attn_dtype_t dtype,
                                 void *stream) {
    g_last_error[0] = 0;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (!x || !w) return fail(ATTN_ERR_ARG, "x or w is NULL");
    if (!aligned16(x) || !aligned16(w)) return fail(ATTN_ERR_ARG, "x or w is not 16-byte aligned");
    if (rows < 0) return fail(ATTN_ERR_ARG, "rows < 0");
    if (width < 8 || width > 8192 || width % 8 != 0)
        return fail(ATTN_ERR_ARG, "width %lld not a multiple of 8 in [8, 8192]", (long long)width);
    if (head < 8 || head % 8 != 0 || width % head != 0)
        return fail(ATTN_ERR_ARG, "head %lld not a multiple of 8 dividing width %lld", (long long)head, (long long)width);
    if (row_stride < width || row_stride % 8 != 0 || row_stride >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_ARG, "row stride %lld not a multiple of 8 in [width, 2^31)", (long long)row_stride);
    if ((cos == nullptr) != (sin == nullptr)) return fail(ATTN_ERR_ARG, "cos and sin must both be given or both NULL");
    if (cos && (!aligned16(cos) || !aligned16(sin))) return fail(ATTN_ERR_ARG, "cos/sin not 16-byte aligned");
    if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(ATTN_ERR_ARG, "eps must be finite and >= 0");
    if (rows >= ((int64_t)1 << 24)) return fail(ATTN_ERR_ARG, "rows %lld >= 2^24", (long long)rows);
    if (rows == 0) return ATTN_OK;
    attn::RowNormRopeLaunch a{};
    a.x = x; a.rows = rows; a.width = width; a.head = head; a.rs = row_stride;
    a.w = w; a.cos = cos; a.sin = sin; a.eps = (float)eps; a.bf16 = dtype == ATTN_BF16;
    return hip_status(attn::launch_row_norm_rope(a, static_cast<hipStream_t>(stream)), "attn_row_norm_rope");
}

int64_t attn_decode_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t d, int64_t max_len) {
    if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || max_len <= 0) return 0;
    return attn::decode_default_splits(batch, hq, hkv, d, max_len);
}

int64_t attn_decode_q_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t max_len, int64_t k_bits) {
    if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || max_len <= 0) return 0;
    if (k_bits != 8 && k_bits != 4 && k_bits != 2) return 0;
    return attn::decode_q_default_splits(batch, hq, hkv, max_len, k_bits);
}

size_t attn_decode_workspace_size(int64_t batch, int64_t hq, int64_t hkv, int64_t d, int64_t max_len,
                                  int64_t splits) {
    if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || max_len <= 0 || splits < 0) return 0;
    if (splits == 0) splits = attn::decode_default_splits(batch, hq, hkv, d, max_len);
    return attn::decode_workspace_bytes(batch, hq, d, splits);
}

static attn_status_t decode_impl(const void *q, const void *k_cache, const void *v_cache, void *out, int64_t batch,
                                 int64_t hq, int64_t hkv, int64_t d, int64_t capacity, const Paging *pg,
                                 const int32_t *lens, const int32_t *pos, int64_t max_len, int64_t max_pos,
                                 const attn_headprep_t *prep, double scale, int64_t splits, void *workspace,
                                 size_t workspace_bytes, attn_dtype_t dtype, void *stream, const char *name) {
    g_last_error[0] = 0;
    attn_status_t st = check_dtype_d(dtype, d);
    if (st) return st;
    if (pg && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "paged pools hold bf16 rows");
    if (batch < 0) return fail(ATTN_ERR_ARG, "negative batch");
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
        return fail(ATTN_ERR_ARG, "hq = %lld must be a positive multiple of hkv = %lld", (long long)hq, (long long)hkv);
    if ((st = check_rows("q", q, hq, d, hq * d))) return st;
    if ((st = check_rows("k_cache", k_cache, hkv, d, hkv * d))) return st;
    if ((st = check_rows("v_cache", v_cache, hkv, d, hkv * d))) return st;
    if ((st = check_rows("out", out, hq, d, hq * d))) return st;
    if (!lens) return fail(ATTN_ERR_ARG, "lens is NULL");
    int64_t rows;                              // cache rows the pointers span
    if (pg) {
        if ((st = check_paging(*pg, max_len, batch))) return st;
        rows = pg->num_pages * pg->page_rows;
    } else {
        if (capacity <= 0 || capacity >= ((int64_t)1 << 31)) return fail(ATTN_ERR_ARG, "capacity %lld outside [1, 2^31)", (long long)capacity);
        if (max_len < 1 || max_len > capacity) return fail(ATTN_ERR_ARG, "max_len %lld outside [1, capacity]", (long long)max_len);
        rows = batch * capacity;
    }
    if (splits < 0 || splits > max_len) return fail(ATTN_ERR_ARG, "splits %lld outside [0, max_len]", (long long)splits);
    if (!std::isfinite(scale) || !(scale > 0.0)) return fail(ATTN_ERR_ARG, "scale must be finite and > 0");
    if (prep) {
        if ((st = check_prep(prep, d, true, false, 0, 0))) return st;
        if (prep->half > 0 && !pos) return fail(ATTN_ERR_ARG, "pos is NULL with a turning HeadPrep");
        if (prep->table_rows >= ((int64_t)1 << 31)) return fail(ATTN_ERR_ARG, "table too large");
        if (prep->half > 0 && (max_pos < 0 || max_pos >= prep->table_rows))
            return fail(ATTN_ERR_ARG, "max_pos %lld outside the table's rows [0, %lld)", (long long)max_pos,
                        (long long)prep->table_rows);
    }
    if (batch == 0) return ATTN_OK;
    if (splits == 0) splits = attn::decode_default_splits(batch, hq, hkv, d, max_len);
    if (splits * batch >= ((int64_t)1 << 31) || splits >= 65536 || batch >= 65536 || hkv * hq >= 65536)
        return fail(ATTN_ERR_ARG, "problem too large for one launch");
    const size_t need = attn::decode_workspace_bytes(batch, hq, d, splits);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
        if (!aligned16(workspace)) return fail(ATTN_ERR_ARG, "workspace is not 16-byte aligned");
    }
    const size_t es = elem_size(dtype);
    const Span so = span(out, batch, hq * d, hq, d, es);
    const Span sw{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
    if (overlap(so, span(q, batch, hq * d, hq, d, es)) || overlap(so, sw) ||
        overlap(so, span(k_cache, rows, hkv * d, hkv, d, es)) ||
        overlap(so, span(v_cache, rows, hkv * d, hkv, d, es)) ||
        (pg && overlap(so, table_span(*pg, batch))))
        return fail(ATTN_ERR_ARG, "out overlaps an input or the workspace");

    attn::DecodeLaunch a{};
    a.q = q; a.k = k_cache; a.v = v_cache; a.out = out;
    a.batch = batch; a.hq = hq; a.hkv = hkv; a.d = d; a.capacity = pg ? pg->page_rows : capacity; a.max_len = max_len;
    a.lens = lens; a.pos = pos;
    if (pg) {
        a.pages = pg->pages; a.page_rows = pg->page_rows; a.max_pages = pg->max_pages; a.num_pages = pg->num_pages;
    }
    a.prep_q = prep != nullptr;
    if (prep) {
        a.qw = prep->qw; a.cos = prep->cos; a.sin = prep->sin; a.half = prep->half;
        // positions past max_pos are out of range for the kernel (NaN rows), like those
        // past the table
        a.table_rows = prep->half > 0 ? max_pos + 1 : prep->table_rows;
        a.pairs = prep->pairs != 0; a.eps = (float)prep->eps;
    }
    a.scale = (float)scale; a.splits = splits; a.work = static_cast<float *>(workspace);
    a.bf16 = dtype == ATTN_BF16;
    return hip_status(attn::launch_decode(a, static_cast<hipStream_t>(stream)), name);
}

attn_status_t attn_decode(const void *q, const void *k_cache, const void *v_cache, void *out, int64_t batch,
                          int64_t hq, int64_t hkv, int64_t d, int64_t capacity, const int32_t *lens,
                          const int32_t *pos, int64_t max_len, int64_t max_pos, const attn_headprep_t *prep,
                          double scale, int64_t splits, void *workspace, size_t workspace_bytes, attn_dtype_t dtype,
                          void *stream) {
    return decode_impl(q, k_cache, v_cache, out, batch, hq, hkv, d, capacity, nullptr, lens, pos, max_len, max_pos, prep,
                       scale, splits, workspace, workspace_bytes, dtype, stream, "attn_decode");
}

attn_status_t attn_decode_paged(const void *q, const void *k_pool, const void *v_pool, void *out, int64_t batch,
                                int64_t hq, int64_t hkv, int64_t d, int64_t num_pages, int64_t page_rows,
                                const int32_t *pages, int64_t max_pages, const int32_t *lens, const int32_t *pos,
                                int64_t max_len, int64_t max_pos, const attn_headprep_t *prep, double scale,
                                int64_t splits, void *workspace, size_t workspace_bytes, attn_dtype_t dtype,
                                void *stream) {
    const Paging pg{pages, page_rows, max_pages, num_pages};
    return decode_impl(q, k_pool, v_pool, out, batch, hq, hkv, d, 0, &pg, lens, pos, max_len, max_pos, prep, scale, splits,
                       workspace, workspace_bytes, dtype, stream, "attn_decode_paged");
}

size_t attn_decode_static_scratch_bytes(void) { return attn::decode_scratch_bytes(); }

attn_status_t attn_decode_static(const void *q, const void *k_cache, const void *v_cache, void *out, int64_t batch,
                                 int64_t hq, int64_t hkv, int64_t d, int64_t capacity, const int32_t *lens,
                                 const int32_t *pos, int64_t max_len, int64_t max_pos, const attn_headprep_t *prep,
                                 double scale, int64_t splits, attn_dtype_t dtype, void *stream) {
    g_last_error[0] = 0;
    const size_t cap = attn::decode_scratch_bytes();
    int64_t s = splits;
    // the split count, and the scratch it needs (decode_impl reports bad arguments; the
    // size is only worked out for sane ones)
    size_t need = 0;
    if (batch > 0 && hq > 0 && hkv > 0 && hq % hkv == 0 && (d == 64 || d == 128) && max_len > 0 && s >= 0) {
        const size_t per_split = attn::decode_workspace_bytes(batch, hq, d, 2) / 2;
        if (s == 0) {
            // the library's choice, lowered until the partials fit (one split needs none)
            s = attn::decode_default_splits(batch, hq, hkv, d, max_len);
            if (s > 1 && (size_t)s * per_split > cap) s = std::max<int64_t>(1, (int64_t)(cap / per_split));
        }
        need = attn::decode_workspace_bytes(batch, hq, d, s);
        if (need > cap)
            return fail(ATTN_ERR_WORKSPACE,
                        "attn_decode_static: %lld splits need %zu bytes of scratch; the library's scratch holds %zu "
                        "(ask for fewer splits, or use attn_decode with a workspace)",
                        (long long)s, need, cap);
    }
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t err = attn::decode_scratch(&ws);
        if (err != hipSuccess) return hip_status(err, "attn_decode_static (scratch address)");
    }
    return decode_impl(q, k_cache, v_cache, out, batch, hq, hkv, d, capacity, nullptr, lens, pos, max_len, max_pos, prep,
                       scale, s, ws, need > 0 ? cap : 0, dtype, stream, "attn_decode_static");
}

attn_status_t attn_kv_quantize(const void *x, int64_t batch, int64_t seq, int64_t heads, int64_t d,
                               int64_t x_row_stride, int64_t bits, uint8_t *codes, float *params,
                               int64_t capacity, int64_t row0, attn_dtype_t dtype, void *stream) {
    g_last_error[0] = 0;
    attn_status_t st = check_dtype_d(dtype, d);
    if (st) return st;
    if (batch < 0 || seq < 0) return fail(ATTN_ERR_ARG, "negative batch or seq");
    if ((st = check_rows("x", x, heads, d, x_row_stride))) return st;
    if (bits != 8 && bits != 4 && bits != 2) return fail(ATTN_ERR_ARG, "bits %lld not 8, 4 or 2", (long long)bits);
    if (!codes || !params) return fail(ATTN_ERR_ARG, "codes or params is NULL");
    if (!aligned16(codes) || !aligned16(params)) return fail(ATTN_ERR_ARG, "codes or params not 16-byte aligned");
    if (capacity <= 0 || capacity >= ((int64_t)1 << 31)) return fail(ATTN_ERR_ARG, "capacity %lld outside [1, 2^31)", (long long)capacity);
    if (row0 < 0 || row0 + seq > capacity)
        return fail(ATTN_ERR_ARG, "rows [%lld, %lld) outside the %lld-row cache", (long long)row0, (long long)(row0 + seq),
                    (long long)capacity);
    if (batch == 0 || seq == 0) return ATTN_OK;
    if (batch * seq * heads >= ((int64_t)1 << 36)) return fail(ATTN_ERR_ARG, "problem too large for one launch");
    const size_t es = elem_size(dtype);
    const Span sx = span(x, batch * seq, x_row_stride, heads, d, es);
    const uintptr_t c0 = reinterpret_cast<uintptr_t>(codes), p0 = reinterpret_cast<uintptr_t>(params);
    const Span sc{c0, c0 + (uintptr_t)(batch * heads * capacity * d * bits / 8)};
    const Span sp{p0, p0 + (uintptr_t)(batch * heads * capacity * 2 * 4)};
    if (overlap(sx, sc) || overlap(sx, sp) || overlap(sc, sp)) return fail(ATTN_ERR_ARG, "x, codes and params overlap");
    attn::KvQuantLaunch a{};
    a.x = x; a.rs = x_row_stride; a.batch = batch; a.seq = seq; a.heads = heads; a.d = d; a.bits = (int)bits;
    a.codes = codes; a.params = params; a.capacity = capacity; a.row0 = row0; a.bf16 = dtype == ATTN_BF16;
    return hip_status(attn::launch_kv_quantize(a, static_cast<hipStream_t>(stream)), "attn_kv_quantize");
}

static attn_status_t decode_q_impl(const void *q, const uint8_t *k_codes, const float *k_params,
                                   const uint8_t *v_codes, const float *v_params, void *out, int64_t batch,
                                   int64_t hq, int64_t hkv, int64_t d, int64_t capacity, const Paging *pg,
                                   int64_t k_bits, int64_t v_bits, const int32_t *lens, const int32_t *pos,
                                   int64_t max_len, int64_t max_pos, const attn_headprep_t *prep, double scale,
                                   int64_t splits,
                                   void *workspace, size_t workspace_bytes, attn_dtype_t dtype, void *stream,
                                   const char *name) {
    g_last_error[0] = 0;
    attn_status_t st = check_dtype_d(dtype, d);
    if (st) return st;
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_q takes bf16 q and out");
    if (batch < 0) return fail(ATTN_ERR_ARG, "negative batch");
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
        return fail(ATTN_ERR_ARG, "hq = %lld must be a positive multiple of hkv = %lld", (long long)hq, (long long)hkv);
    if (!((k_bits == 8 && v_bits == 8) || (k_bits == 4 && v_bits == 4) || (k_bits == 4 && v_bits == 2) ||
          (k_bits == 2 && v_bits == 2)))
        return fail(ATTN_ERR_ARG, "bits (%lld, %lld) not (8, 8), (4, 4), (4, 2) or (2, 2)", (long long)k_bits,
                    (long long)v_bits);
    if ((st = check_rows("q", q, hq, d, hq * d))) return st;
    if ((st = check_rows("out", out, hq, d, hq * d))) return st;
    if (!k_codes || !k_params || !v_codes || !v_params) return fail(ATTN_ERR_ARG, "a cache pointer is NULL");
    if (!aligned16(k_codes) || !aligned16(k_params) || !aligned16(v_codes) || !aligned16(v_params))
        return fail(ATTN_ERR_ARG, "cache pointers must be 16-byte aligned");
    if (!lens) return fail(ATTN_ERR_ARG, "lens is NULL");
    int64_t units, urows;                      // the caches' units (sequences or pages) and rows per unit
    if (pg) {
        if ((st = check_paging(*pg, max_len, batch))) return st;
        units = pg->num_pages; urows = pg->page_rows;
    } else {
        if (capacity <= 0 || capacity >= ((int64_t)1 << 31)) return fail(ATTN_ERR_ARG, "capacity %lld outside [1, 2^31)", (long long)capacity);
        if (max_len < 1 || max_len > capacity) return fail(ATTN_ERR_ARG, "max_len %lld outside [1, capacity]", (long long)max_len);
        units = batch; urows = capacity;
    }
    if (splits < 0 || splits > max_len) return fail(ATTN_ERR_ARG, "splits %lld outside [0, max_len]", (long long)splits);
    if (!std::isfinite(scale) || !(scale > 0.0)) return fail(ATTN_ERR_ARG, "scale must be finite and > 0");
    if (prep) {
        if ((st = check_prep(prep, d, true, false, 0, 0))) return st;
        if (prep->half > 0 && !pos) return fail(ATTN_ERR_ARG, "pos is NULL with a turning HeadPrep");
        if (prep->table_rows >= ((int64_t)1 << 31)) return fail(ATTN_ERR_ARG, "table too large");
        if (prep->half > 0 && (max_pos < 0 || max_pos >= prep->table_rows))
            return fail(ATTN_ERR_ARG, "max_pos %lld outside the table's rows [0, %lld)", (long long)max_pos,
                        (long long)prep->table_rows);
    }
    if (batch == 0) return ATTN_OK;
    if (splits == 0) splits = attn::decode_q_default_splits(batch, hq, hkv, max_len, k_bits);
    if (splits * batch >= ((int64_t)1 << 31) || splits >= 65536 || batch >= 65536 || hkv * hq >= 65536 ||
        units * hkv * urows * d >= ((int64_t)1 << 40) || units * hkv * urows >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_ARG, "problem too large for one launch");
    const size_t need = attn::decode_workspace_bytes(batch, hq, d, splits);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
        if (!aligned16(workspace)) return fail(ATTN_ERR_ARG, "workspace is not 16-byte aligned");
    }
    const Span so = span(out, batch, hq * d, hq, d, 2);
    const Span sw{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
    auto bytes_span = [](const void *ptr, int64_t n) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(ptr);
        return Span{a, a + (uintptr_t)n};
    };
    const int64_t rows = units * hkv * urows;
    if (overlap(so, span(q, batch, hq * d, hq, d, 2)) || overlap(so, sw) ||
        overlap(so, bytes_span(k_codes, rows * d * k_bits / 8)) || overlap(so, bytes_span(v_codes, rows * d * v_bits / 8)) ||
        overlap(so, bytes_span(k_params, rows * 8)) || overlap(so, bytes_span(v_params, rows * 8)) ||
        (pg && overlap(so, table_span(*pg, batch))))
        return fail(ATTN_ERR_ARG, "out overlaps an input or the workspace");

    attn::DecodeLaunch a{};
    a.q = q; a.k = k_codes; a.v = v_codes; a.out = out;
    a.batch = batch; a.hq = hq; a.hkv = hkv; a.d = d; a.capacity = urows; a.max_len = max_len;
    a.lens = lens; a.pos = pos;
    if (pg) {
        a.pages = pg->pages; a.page_rows = pg->page_rows; a.max_pages = pg->max_pages; a.num_pages = pg->num_pages;
    }
    a.prep_q = prep != nullptr;
    if (prep) {
        a.qw = prep->qw; a.cos = prep->cos; a.sin = prep->sin; a.half = prep->half;
        // positions past max_pos are out of range for the kernel (NaN rows), like those
        // past the table
        a.table_rows = prep->half > 0 ? max_pos + 1 : prep->table_rows;
        a.pairs = prep->pairs != 0; a.eps = (float)prep->eps;
    }
    a.scale = (float)scale; a.splits = splits; a.work = static_cast<float *>(workspace);
    a.bf16 = true;
    a.kpar = k_params; a.vpar = v_params; a.kbits = (int)k_bits; a.vbits = (int)v_bits;
    return hip_status(attn::launch_decode(a, static_cast<hipStream_t>(stream)), name);
}

attn_status_t attn_decode_q(const void *q, const uint8_t *k_codes, const float *k_params, const uint8_t *v_codes,
                            const float *v_params, void *out, int64_t batch, int64_t hq, int64_t hkv, int64_t d,
                            int64_t capacity, int64_t k_bits, int64_t v_bits, const int32_t *lens,
                            const int32_t *pos, int64_t max_len, int64_t max_pos, const attn_headprep_t *prep,
                            double scale, int64_t splits, void *workspace, size_t workspace_bytes, attn_dtype_t dtype,
                            void *stream) {
    return decode_q_impl(q, k_codes, k_params, v_codes, v_params, out, batch, hq, hkv, d, capacity, nullptr, k_bits,
                         v_bits, lens, pos, max_len, max_pos, prep, scale, splits, workspace, workspace_bytes, dtype, stream,
                         "attn_decode_q");
}

attn_status_t attn_decode_q_paged(const void *q, const uint8_t *k_codes, const float *k_params,
                                  const uint8_t *v_codes, const float *v_params, void *out, int64_t batch, int64_t hq,
                                  int64_t hkv, int64_t d, int64_t num_pages, int64_t page_rows, int64_t k_bits,
                                  int64_t v_bits, const int32_t *pages, int64_t max_pages, const int32_t *lens,
                                  const int32_t *pos, int64_t max_len, int64_t max_pos,
                                  const attn_headprep_t *prep, double scale, int64_t splits, void *workspace,
                                  size_t workspace_bytes, attn_dtype_t dtype, void *stream) {
    const Paging pg{pages, page_rows, max_pages, num_pages};
    return decode_q_impl(q, k_codes, k_params, v_codes, v_params, out, batch, hq, hkv, d, 0, &pg, k_bits, v_bits, lens,
                         pos, max_len, max_pos, prep, scale, splits, workspace, workspace_bytes, dtype, stream,
                         "attn_decode_q_paged");
}

double attn_key_bound(const float *kw, int64_t d) {
    if (!kw || d <= 0) return -1.0;
    double m = 0.0;
    for (int64_t i = 0; i < d; ++i) {
        if (!std::isfinite(kw[i])) return std::nan("");
        m = std::max(m, (double)std::fabs(kw[i]));
    }
    return std::sqrt((double)d) * m * (1.0 + 1.0 / 128);
}

}  // extern "C"
