// decode_common.h -- pieces shared by the decode kernels (bf16 / f32 caches in
// decode.hip, quantised caches in kvq.hip): block geometry, the parameter block, the
// query's HeadPrep prologue, the merge of the waves' online-softmax states, and the LDS
// layout of a chunk of 16 bf16 cache rows.  Internal to libattn.
#pragma once

#include "common.h"
#include "kernels.h"

namespace attn {

struct DecodeParams {
    const void *q; const void *k; const void *v;
    float *work;
    void *out;                  // written directly when there is a single split
    bool direct, check_pos;
    int64_t batch, hq, hkv, capacity, max_len, per_split, splits;
    const int32_t *lens, *pos;
    const float *qw, *cos, *sin;
    int half, table_rows, group, ngroups;
    float eps, C;
    bool prep_q, pairs;
    const float *kpar, *vpar;   // quantised caches: (lo, step) of every cached head
    // Paged pool (pages != NULL): key j of sequence b lives in pool page
    // pages[b max_pages + j / page_rows], row j % page_rows; page_rows = 2^page_shift.
    const int32_t *pages;
    int page_shift, max_pages, num_pages;
};

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kChunk = 16;            // keys per wave step (the 16 rows of one MFMA)
constexpr float kRaiseAbove = 8.0f;   // base-2 headroom before the running max moves
constexpr int64_t kCUs = 256;         // compute units of one MI355X

// Block coordinates: the kv-head groups of one (sequence, split) are consecutive block
// ids, so the blocks reading the same cache rows are dealt to different XCDs together.
struct BlockCoord {
    int split, kvh, grp, b;
};
__device__ __forceinline__ BlockCoord block_coord(const DecodeParams &p) {
    BlockCoord c;
    c.kvh = blockIdx.x / p.ngroups;
    c.grp = blockIdx.x % p.ngroups;
    c.split = blockIdx.y;
    c.b = blockIdx.z;
    return c;
}

// Where key `key` (< max_len) of sequence b lives: the unit (sequence b of a contiguous
// cache, or the pool page holding it) and the row within it.  A page id outside the pool
// is replaced by page 0 (every read stays inside the pool) and sets `bad`.
struct CacheSlot {
    int unit, row;
};
__device__ __forceinline__ CacheSlot cache_slot(const DecodeParams &p, int b, int key, bool &bad) {
    if (!p.pages) return CacheSlot{b, key};
    int id = p.pages[(int64_t)b * p.max_pages + (key >> p.page_shift)];
    if ((unsigned)id >= (unsigned)p.num_pages) {
        bad = true;
        id = 0;
    }
    return CacheSlot{id, key & ((1 << p.page_shift) - 1)};
}

// Rows per unit: the capacity of a contiguous cache, or the page size.
__device__ __forceinline__ int64_t unit_rows(const DecodeParams &p) {
    return p.pages ? ((int64_t)1 << p.page_shift) : p.capacity;
}

// Load the block's q heads, RMS-normalise with qw and turn at table row pos[b] (when
// prep_q); leaves the prepped rows in qh (f32).  Every thread of the block takes part;
// `part` is LDS scratch of kThreads / 64 floats.
template <bool BF16, int D, int GB>
__device__ void q_prologue(const DecodeParams &p, int b, int h0, int nh, float (*qs)[D], float (*qh)[D],
                           float *part) {
    const int tid = threadIdx.x, w = tid / 64;
    for (int idx = tid; idx < GB * D; idx += kThreads) {
        const int i = idx / D, e = idx % D;
        float x = 0.f;
        if (i < nh) {
            const int64_t off = ((int64_t)b * p.hq + h0 + i) * D + e;
            x = BF16 ? bf16_bits_to_f32(static_cast<const uint16_t *>(p.q)[off])
                     : static_cast<const float *>(p.q)[off];
        }
        qs[i][e] = x;
    }
    __syncthreads();
    if (p.prep_q) {
        // 256 threads = GB heads x (256 / GB) lanes; each lane sums D*GB/256 squares.
        constexpr int LPH = kThreads / GB;
        constexpr int EPL = D / LPH > 0 ? D / LPH : 1;
        const int i = tid / LPH, li = tid % LPH;
        float ss = 0.f;
        if (li * EPL < D)
            for (int e = li * EPL; e < li * EPL + EPL; ++e) ss += qs[i][e] * qs[i][e];
        ss = sum_lanes<(LPH < 64 ? LPH : 64)>(ss);
        __syncthreads();
        if (LPH > 64) {   // reduce across the waves of one head (part: kThreads / 64 floats)
            if (tid % 64 == 0) part[w] = ss;
            __syncthreads();
            ss = 0.f;
            for (int j = 0; j < LPH / 64; ++j) ss += part[(i * LPH) / 64 + j];
        }
        const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / D) + p.eps);
        if (li * EPL < D)
            for (int e = li * EPL; e < li * EPL + EPL; ++e) qs[i][e] = qs[i][e] * inv * p.qw[e];
        __syncthreads();
        const int pr = p.half > 0 ? p.pos[b] : 0;     // pos may be NULL without a turn
        const int prow = pr < 0 ? 0 : (pr >= p.table_rows ? p.table_rows - 1 : pr);
        for (int idx = tid; idx < GB * D; idx += kThreads) {
            const int hh = idx / D, e = idx % D;
            float y = qs[hh][e];
            if (p.pairs) {       // adjacent pairs (2j, 2j + 1), table entry j
                const int j = e >> 1;
                if (j < p.half) {
                    const float c = p.cos[(int64_t)prow * p.half + j], s = p.sin[(int64_t)prow * p.half + j];
                    y = (e & 1) ? qs[hh][e] * c + qs[hh][e - 1] * s : qs[hh][e] * c - qs[hh][e + 1] * s;
                }
            } else if (e < p.half) {
                const float c = p.cos[(int64_t)prow * p.half + e], s = p.sin[(int64_t)prow * p.half + e];
                y = qs[hh][e] * c - qs[hh][e + p.half] * s;
            } else if (e < 2 * p.half) {
                const int f = e - p.half;
                const float c = p.cos[(int64_t)prow * p.half + f], s = p.sin[(int64_t)prow * p.half + f];
                y = qs[hh][e] * c + qs[hh][f] * s;
            }
            qh[hh][e] = y;
        }
    } else {
        for (int idx = tid; idx < GB * D; idx += kThreads) qh[idx / D][idx % D] = qs[idx / D][idx % D];
    }
    __syncthreads();
}

// Merge the waves' states (wm, wl, wo in LDS, written before a block barrier).  With
// several splits, write the block's partial (a[d], m, l) of each of its q heads to the
// workspace; with one split, write the output rows themselves (a / l, zeros for an
// empty row, NaN for a row with invalid lens or pos).
template <bool BF16, int D, int GB>
__device__ void write_partial(const DecodeParams &p, int split, int b, int h0, int nh, const float (*wm)[GB],
                              const float (*wl)[GB], const float (*wo)[GB][D], bool page_bad = false) {
    const int64_t stride = (int64_t)D + 2;
    bool bad = page_bad;
    if (p.direct) {
        const int len = p.lens[b];
        bad = bad || len < 0 || len > p.max_len;
        if (p.check_pos) {
            const int pr = p.pos[b];
            bad = bad || pr < 0 || pr >= p.table_rows;
        }
    }
    for (int idx = threadIdx.x; idx < nh * D; idx += kThreads) {
        const int i = idx / D, e = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, wm[ww][i]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                const float f = fast_exp2(wm[ww][i] - M);
                L += wl[ww][i] * f;
                A += wo[ww][i][e] * f;
            }
        }
        const int64_t row = (int64_t)b * p.hq + h0 + i;
        if (p.direct) {
            float y = L > 0.f ? A / L : 0.f;
            if (bad) y = __builtin_nanf("");
            if constexpr (BF16) {
                f32x2 v2 = {y, 0.f};
                bf16x2 hv = __builtin_convertvector(v2, bf16x2);
                static_cast<uint16_t *>(p.out)[row * D + e] = (uint16_t)(__builtin_bit_cast(uint32_t, hv) & 0xFFFFu);
            } else {
                static_cast<float *>(p.out)[row * D + e] = y;
            }
        } else {
            float *dst = p.work + ((int64_t)split * p.batch * p.hq + row) * stride;
            dst[e] = A;
            if (e == 0) {
                dst[D] = M;
                dst[D + 1] = page_bad ? __builtin_nanf("") : L;   // the merge turns a NaN sum into NaN rows
            }
        }
    }
}

// ---------------------------------------------------------------------------------
// bf16 caches.

template <int D>
struct DecGeo {
    static constexpr int kRow = 2 * D;               // bytes of one cache row of one kv head
    static constexpr int kCpr = kRow / 16;           // 16-byte chunks per row
    static constexpr int kRpi = 64 / kCpr;           // rows per 64-lane load
    static constexpr int kLoads = kChunk / kRpi;     // 16-byte loads per lane per chunk, each of K and V
    static constexpr int kKMfma = D / 32;            // S^T MFMAs per chunk (per q part)
    static constexpr int kNT = D / 16;               // 16-row d tiles of O^T
    static constexpr int kBuf = kChunk * kRow;       // LDS bytes of one chunk of K (or of V)
};

// LDS slot of 16-byte chunk c of row `row` (0..15) of a K or V chunk.  The swizzles make
// the reads conflict-free: the K fragment reads of 16 lanes (16 rows, one chunk each)
// and the transposing V reads of 32 lanes (8 rows x 32 bytes) touch 64 distinct banks.
template <int D>
__device__ __forceinline__ int kslot(int row, int c) {
    return c ^ (D == 128 ? row : row >> 1);
}
template <int D>
__device__ __forceinline__ int vslot(int row, int c) {
    return c ^ (D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3));
}

}  // namespace

// Parameter block of a decode launch (geometry, splits, HeadPrep) from its ABI record.
DecodeParams make_decode_params(const DecodeLaunch &a);
// The split-merge pass (only when a.splits > 1).
hipError_t launch_decode_merge(const DecodeLaunch &a, hipStream_t stream);

}  // namespace attn
