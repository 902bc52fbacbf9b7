// prep.hip -- HeadPrep kernel (gizml:netops reference page, Types > HeadPrep and
// Functions > headPrepInPlace).
//
// One head of d values is one work unit: over its RMS (eps under the root), times
// its norm weight, then values e < half turned with e + half by the cos/sin row of
// the token's sequence position.  q and k units share one launch.
//
// The pass is HBM-bound (read and write each value once), so the layout is chosen for
// coalescing: d/8 consecutive lanes own one head, lane i holding the 4 values at
// 4i.. and the 4 values at d/2 + 4i.., so each wave reads 2 x 64 contiguous 8-byte
// (bf16) or 16-byte (f32) pieces and, when half = d/2, every turned pair sits in one
// lane.  Other halves go through LDS.  Adjacent pairs (2i, 2i + 1: FLUX.3's layout)
// always sit in one lane, whatever half is.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kPrepThreads = 256;

struct PrepParams {
    const void *q_src; void *q_dst; int64_t q_src_rs, q_dst_rs; int64_t hq;
    const void *k_src; void *k_dst; int64_t k_src_rs, k_dst_rs; int64_t hkv;
    int64_t q_src_bs, q_dst_bs, k_src_bs, k_dst_bs;
    int64_t seq, pos0, n_q_units, n_units;
    const float *qw, *kw, *cos, *sin;
    int half;
    float eps;
    PageMap k_pages;            // pages != NULL: k rows go to pool rows (see PrepLaunch)
    int64_t k_row0;
    const int32_t *past;        // per-sequence positions (see PrepLaunch)
    int64_t past_max;
};

// Turn the adjacent pairs (e, e + 1), e even, of 4 values starting at e0 (a multiple of
// 4) by table entries e / 2 < half of row `crow` / `srow`.
__device__ __forceinline__ void turn_pairs4(float (&x)[4], int e0, int half, const float *crow,
                                            const float *srow) {
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
        const int j = (e0 + i) / 2;
        if (j < half) {
            const float c = crow[j], s = srow[j], a = x[i], b = x[i + 1];
            x[i] = a * c - b * s;
            x[i + 1] = b * c + a * s;
        }
    }
}

template <bool BF16>
__device__ __forceinline__ void load4(const void *base, int64_t off, float (&x)[4]) {
    if constexpr (BF16) {
        const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + off);
        unpack_bf16x2(w.x, x[0], x[1]);
        unpack_bf16x2(w.y, x[2], x[3]);
    } else {
        const float4 w = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off);
        x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
    }
}

template <bool BF16>
__device__ __forceinline__ void store4(void *base, int64_t off, const float (&x)[4]) {
    if constexpr (BF16) {
        uint2 w;
        w.x = pack_bf16x2(x[0], x[1]);
        w.y = pack_bf16x2(x[2], x[3]);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(base) + off) = w;
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(base) + off) =
            make_float4(x[0], x[1], x[2], x[3]);
    }
}

// One head of the launch: where it is read and written, and its values in flight.
template <bool BF16, int D, int MODE>
struct PrepUnit {
    bool valid;
    const void *src;
    void *dst;
    int64_t src_off, dst_off, posrow;   // dst_off < 0: a page outside the pool, not written
    const float *w;
    float lo[4], hi[4];
    float4 wl, wh, cq, sq;

    // IX: the integer type of the unit index arithmetic (32-bit when every unit index
    // fits: two divisions then cost a few instructions each instead of a long 64-bit
    // sequence, for every lane of every head).
    template <typename IX>
    __device__ __forceinline__ void locate(const PrepParams &p, int64_t unit) {
        valid = unit < p.n_units;
        const bool is_q = unit < p.n_q_units;
        const IX uu = (IX)(valid ? (is_q ? unit : unit - p.n_q_units) : 0);
        const IX heads = (IX)(is_q ? p.hq : p.hkv);
        const IX rowi = uu / heads;
        const IX hi_ = uu - rowi * heads;
        const IX bbi = rowi / (IX)p.seq;
        const int64_t bb = (int64_t)bbi, hh = (int64_t)hi_;
        // the sequence's first position: pos0, or its own past[b] (0 when out of range,
        // and then its key rows are not written)
        int64_t first = p.pos0, krow0 = p.k_row0;
        bool seq_ok = true;
        if (p.past) {
            const int v = p.past[bb];
            seq_ok = v >= 0 && v <= p.past_max;
            first = seq_ok ? v : 0;
            krow0 = first;
        }
        const int64_t t = (int64_t)(rowi - bbi * (IX)p.seq);
        if (is_q) {
            const int64_t h = hh;
            src = p.q_src; dst = p.q_dst; w = p.qw;
            src_off = bb * p.q_src_bs + t * p.q_src_rs + h * D;
            dst_off = bb * p.q_dst_bs + t * p.q_dst_rs + h * D;
        } else {
            const int64_t h = hh;
            src = p.k_src; dst = p.k_dst; w = p.kw;
            src_off = bb * p.k_src_bs + t * p.k_src_rs + h * D;
            dst_off = bb * p.k_dst_bs + ((p.past ? krow0 : 0) + t) * p.k_dst_rs + h * D;
            if (p.k_pages.pages && valid) {
                bool bad = false;
                const int64_t prow = pool_row(p.k_pages, (int)bb, krow0 + t, bad);
                dst_off = bad ? -1 : prow * p.k_dst_rs + h * D;
            }
            if (!seq_ok) dst_off = -1;
        }
        posrow = first + t;
    }

    // The weights, (split halves, half = D/2) the lane's table entries and the values,
    // all requested before anything waits: one memory round trip per head.
    __device__ __forceinline__ void load(const PrepParams &p, int e_lo, int e_hi) {
        wl = wh = cq = sq = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = hi[i] = 0.f;
        if (valid) {
            wl = *reinterpret_cast<const float4 *>(w + e_lo);
            wh = *reinterpret_cast<const float4 *>(w + e_hi);
            if constexpr (MODE == 1) {
                cq = *reinterpret_cast<const float4 *>(p.cos + posrow * (D / 2) + e_lo);
                sq = *reinterpret_cast<const float4 *>(p.sin + posrow * (D / 2) + e_lo);
            }
            load4<BF16>(src, src_off + e_lo, lo);
            load4<BF16>(src, src_off + e_hi, hi);
        }
    }

    // Norm, weight, turn, store.  `stage` (MODE 2): this head's D floats of LDS; every
    // thread of the block must call this together then (it holds a block barrier).
    template <int LPH>
    __device__ __forceinline__ void finish(const PrepParams &p, int e_lo, int e_hi, float *stage) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += lo[i] * lo[i] + hi[i] * hi[i];
        ss = sum_lanes<LPH>(ss);
        const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / D) + p.eps);
        if (valid) {
            lo[0] = lo[0] * inv * wl.x; lo[1] = lo[1] * inv * wl.y;
            lo[2] = lo[2] * inv * wl.z; lo[3] = lo[3] * inv * wl.w;
            hi[0] = hi[0] * inv * wh.x; hi[1] = hi[1] * inv * wh.y;
            hi[2] = hi[2] * inv * wh.z; hi[3] = hi[3] * inv * wh.w;
        }
        if constexpr (MODE == 3) {
            if (valid) {
                const float *crow = p.cos + posrow * p.half, *srow = p.sin + posrow * p.half;
                turn_pairs4(lo, e_lo, p.half, crow, srow);
                turn_pairs4(hi, e_hi, p.half, crow, srow);
            }
        } else if constexpr (MODE == 1) {
            if (valid) {
                const float cc[4] = {cq.x, cq.y, cq.z, cq.w}, sc[4] = {sq.x, sq.y, sq.z, sq.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a = lo[i], b = hi[i];
                    lo[i] = a * cc[i] - b * sc[i];
                    hi[i] = b * cc[i] + a * sc[i];
                }
            }
        } else if constexpr (MODE == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                stage[e_lo + i] = lo[i];
                stage[e_hi + i] = hi[i];
            }
            __syncthreads();
            if (valid) {
                const int half = p.half;
                const float *crow = p.cos + posrow * half;
                const float *srow = p.sin + posrow * half;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int e = i < 4 ? e_lo + i : e_hi + i - 4;
                    float y = stage[e];
                    if (e < half) {
                        y = stage[e] * crow[e] - stage[e + half] * srow[e];
                    } else if (e < 2 * half) {
                        const int f = e - half;
                        y = stage[e] * crow[f] + stage[f] * srow[f];
                    }
                    if (i < 4) lo[i] = y; else hi[i - 4] = y;
                }
            }
        }
        if (valid && dst_off >= 0) {
            store4<BF16>(dst, dst_off + e_lo, lo);
            store4<BF16>(dst, dst_off + e_hi, hi);
        }
    }
};

// MODE 0: no turn (half = 0); MODE 1: half = d/2, pairs in-lane; MODE 2: any half, via LDS;
// MODE 3: adjacent pairs, any half, in-lane.  A group of D/8 lanes takes U consecutive
// heads, whose loads are all in flight together (U = 1 for MODE 2, whose LDS stage holds
// one head per lane group).
template <bool BF16, int D, int MODE, int U, bool NARROW>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const PrepParams p) {
    constexpr int LPH = D / 8;                  // lanes per head
    constexpr int HPB = kPrepThreads / LPH;     // lane groups per block
    static_assert(MODE != 2 || U == 1, "the LDS stage holds one head per lane group");
    __shared__ float stage[MODE == 2 ? HPB * D : 1];

    const int li = threadIdx.x % LPH;
    const int hb = threadIdx.x / LPH;
    const int e_lo = 4 * li, e_hi = D / 2 + 4 * li;
    PrepUnit<BF16, D, MODE> units[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t unit = ((int64_t)blockIdx.x * HPB + hb) * U + u;
        if constexpr (NARROW)
            units[u].template locate<uint32_t>(p, unit);
        else
            units[u].template locate<int64_t>(p, unit);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) units[u].load(p, e_lo, e_hi);
#pragma unroll
    for (int u = 0; u < U; ++u) units[u].template finish<LPH>(p, e_lo, e_hi, stage + (MODE == 2 ? hb * D : 0));
}

template <bool BF16, int D>
hipError_t launch_prep_d(const PrepParams &p, int mode, hipStream_t stream) {
    constexpr int HPB = kPrepThreads / (D / 8);
    // Heads per lane group for the modes without the LDS stage: 1 (4 heads per group, all
    // in flight together, measured slower on the 16 MiB prefill keys).
    constexpr int U = 1;
    const int64_t blocks1 = (p.n_units + HPB - 1) / HPB;
    const int64_t blocksU = (p.n_units + HPB * U - 1) / (HPB * U);
    if (blocks1 == 0) return hipSuccess;
    // 32-bit unit arithmetic when every unit index (and so every row and head index) fits
    const bool narrow = p.n_units + HPB * U < ((int64_t)1 << 32);
    if (narrow) {
        if (mode == 0)
            hipLaunchKernelGGL((prep_kernel<BF16, D, 0, U, true>), dim3(blocksU), dim3(kPrepThreads), 0, stream, p);
        else if (mode == 1)
            hipLaunchKernelGGL((prep_kernel<BF16, D, 1, U, true>), dim3(blocksU), dim3(kPrepThreads), 0, stream, p);
        else if (mode == 2)
            hipLaunchKernelGGL((prep_kernel<BF16, D, 2, 1, true>), dim3(blocks1), dim3(kPrepThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((prep_kernel<BF16, D, 3, U, true>), dim3(blocksU), dim3(kPrepThreads), 0, stream, p);
    } else {
        if (mode == 0)
            hipLaunchKernelGGL((prep_kernel<BF16, D, 0, U, false>), dim3(blocksU), dim3(kPrepThreads), 0, stream, p);
        else if (mode == 1)
            hipLaunchKernelGGL((prep_kernel<BF16, D, 1, U, false>), dim3(blocksU), dim3(kPrepThreads), 0, stream, p);
        else if (mode == 2)
            hipLaunchKernelGGL((prep_kernel<BF16, D, 2, 1, false>), dim3(blocks1), dim3(kPrepThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((prep_kernel<BF16, D, 3, U, false>), dim3(blocksU), dim3(kPrepThreads), 0, stream, p);
    }
    return hipGetLastError();
}

// Row copy (16 bytes per lane, grid-stride): row t of sequence b.
// With a page map, row t of sequence b goes to pool row pool_row(pages, b, row0 + t)
// (rows dst_rs bytes apart), and rows whose page id lies outside the pool are skipped.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint8_t *src, uint8_t *dst, int64_t src_bs,
                                                        int64_t src_rs, int64_t dst_bs, int64_t dst_rs,
                                                        int64_t rows, int64_t row_bytes, int64_t total16,
                                                        const PageMap pages, int64_t row0, const int32_t *past,
                                                        int64_t past_max) {
    const int64_t per_row = row_bytes / 16;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total16; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t rr = i / per_row, c = i % per_row;
        const int64_t bb = rr / rows, t = rr % rows;
        int64_t r0 = row0, doff0 = 0;
        if (past) {                         // the sequence's own first row
            const int v = past[bb];
            if (v < 0 || v > past_max) continue;
            r0 = v;
            doff0 = v;
        }
        const uint4 v = *reinterpret_cast<const uint4 *>(src + bb * src_bs + t * src_rs + 16 * c);
        int64_t doff = bb * dst_bs + (doff0 + t) * dst_rs;
        if (pages.pages) {
            bool bad = false;
            const int64_t prow = pool_row(pages, (int)bb, r0 + t, bad);
            if (bad) continue;
            doff = prow * dst_rs;
        }
        *reinterpret_cast<uint4 *>(dst + doff + 16 * c) = v;
    }
}

// Whole-row norm and per-head rotary (gizml:netops, Functions > rowNormRopeInto): one
// block per row.  A unit is 4 values at h * head + 4i and the 4 at h * head + head / 2 +
// 4i (the same lane layout as the HeadPrep kernel, so the turned pairs sit in one lane);
// thread t owns units t, t + 256, ...; the row's sum of squares is reduced over the block.
struct RowNormParams {
    void *x; int64_t rs;
    int width, head;
    const float *w, *cos, *sin;
    float eps;
};

template <bool BF16, int NPT>
__global__ __launch_bounds__(256) void row_norm_rope_kernel(const RowNormParams p) {
    __shared__ float part[4];
    const int64_t r = blockIdx.x;
    const int units = p.width / 8, hu = p.head / 8, halfh = p.head / 2;
    const int64_t base = r * p.rs;
    float lo[NPT][4], hi[NPT][4];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int u = threadIdx.x + 256 * k;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[k][i] = hi[k][i] = 0.f;
        if (u < units) {
            const int e = (u / hu) * p.head + 4 * (u % hu);
            load4<BF16>(p.x, base + e, lo[k]);
            load4<BF16>(p.x, base + e + halfh, hi[k]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += lo[k][i] * lo[k][i] + hi[k][i] * hi[k][i];
    }
    ss = sum_lanes<64>(ss);
    if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = ss;
    __syncthreads();
    ss = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = 1.0f / __builtin_sqrtf(ss / (float)p.width + p.eps);
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int u = threadIdx.x + 256 * k;
        if (u >= units) continue;
        const int h = u / hu, li = u % hu;
        const int e = h * p.head + 4 * li;
        const float4 wl = *reinterpret_cast<const float4 *>(p.w + e);
        const float4 wh = *reinterpret_cast<const float4 *>(p.w + e + halfh);
        const float wlo[4] = {wl.x, wl.y, wl.z, wl.w}, whi[4] = {wh.x, wh.y, wh.z, wh.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo[k][i] = lo[k][i] * inv * wlo[i];
            hi[k][i] = hi[k][i] * inv * whi[i];
        }
        if (p.cos) {
            // pair h * head / 2 + d of the row's table entry, d = 4 li + i
            const int64_t t = r * (p.width / 2) + h * halfh + 4 * li;
            const float4 c = *reinterpret_cast<const float4 *>(p.cos + t);
            const float4 sn = *reinterpret_cast<const float4 *>(p.sin + t);
            const float cc[4] = {c.x, c.y, c.z, c.w}, sc[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = lo[k][i], b = hi[k][i];
                lo[k][i] = a * cc[i] - b * sc[i];
                hi[k][i] = b * cc[i] + a * sc[i];
            }
        }
        store4<BF16>(p.x, base + e, lo[k]);
        store4<BF16>(p.x, base + e + halfh, hi[k]);
    }
}

template <bool BF16>
void launch_row_norm_npt(const RowNormParams &p, int64_t rows, hipStream_t stream) {
    const int units = p.width / 8;
    const dim3 grid((unsigned)rows);
    if (units <= 256)
        hipLaunchKernelGGL((row_norm_rope_kernel<BF16, 1>), grid, dim3(256), 0, stream, p);
    else if (units <= 512)
        hipLaunchKernelGGL((row_norm_rope_kernel<BF16, 2>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((row_norm_rope_kernel<BF16, 4>), grid, dim3(256), 0, stream, p);
}

}  // namespace

hipError_t launch_row_norm_rope(const RowNormRopeLaunch &a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    RowNormParams p;
    p.x = a.x; p.rs = a.rs; p.width = (int)a.width; p.head = (int)a.head;
    p.w = a.w; p.cos = a.cos; p.sin = a.sin; p.eps = a.eps;
    if (a.bf16) launch_row_norm_npt<true>(p, a.rows, stream); else launch_row_norm_npt<false>(p, a.rows, stream);
    return hipGetLastError();
}

hipError_t launch_copy_rows(const CopyRowsLaunch &a, hipStream_t stream) {
    const int64_t row_bytes = a.row_elems * a.elem;
    const int64_t total16 = a.batch * a.rows * (row_bytes / 16);
    if (total16 == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total16 + 255) / 256, 4096);
    hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(a.src), static_cast<uint8_t *>(a.dst), a.src_bs * a.elem,
                       a.src_rs * a.elem, a.dst_bs * a.elem, a.dst_rs * a.elem, a.rows, row_bytes, total16,
                       a.dst_pages, a.dst_row0, a.past, a.past_max);
    return hipGetLastError();
}

hipError_t launch_prep(const PrepLaunch &a, hipStream_t stream) {
    PrepParams p;
    p.q_src = a.q_src; p.q_dst = a.q_dst; p.q_src_rs = a.q_src_rs; p.q_dst_rs = a.q_dst_rs;
    p.hq = a.q_src ? a.hq : 1;
    p.k_src = a.k_src; p.k_dst = a.k_dst; p.k_src_rs = a.k_src_rs; p.k_dst_rs = a.k_dst_rs;
    p.hkv = a.k_src ? a.hkv : 1;
    p.q_src_bs = a.q_src_bs ? a.q_src_bs : a.seq * a.q_src_rs;
    p.q_dst_bs = a.q_dst_bs ? a.q_dst_bs : a.seq * a.q_dst_rs;
    p.k_src_bs = a.k_src_bs ? a.k_src_bs : a.seq * a.k_src_rs;
    p.k_dst_bs = a.k_dst_bs ? a.k_dst_bs : a.seq * a.k_dst_rs;
    p.seq = a.seq;
    p.pos0 = a.pos0;
    p.n_q_units = a.q_src ? a.batch * a.seq * a.hq : 0;
    p.n_units = p.n_q_units + (a.k_src ? a.batch * a.seq * a.hkv : 0);
    p.qw = a.qw; p.kw = a.kw; p.cos = a.cos; p.sin = a.sin;
    p.half = (int)a.half;
    p.eps = a.eps;
    p.k_pages = a.k_pages;
    p.k_row0 = a.k_row0;
    p.past = a.past;
    p.past_max = a.past_max;
    const int mode = a.half == 0 ? 0 : (a.pairs ? 3 : (2 * a.half == a.d ? 1 : 2));
    if (a.d == 64)
        return a.bf16 ? launch_prep_d<true, 64>(p, mode, stream) : launch_prep_d<false, 64>(p, mode, stream);
    return a.bf16 ? launch_prep_d<true, 128>(p, mode, stream) : launch_prep_d<false, 128>(p, mode, stream);
}

}  // namespace attn
