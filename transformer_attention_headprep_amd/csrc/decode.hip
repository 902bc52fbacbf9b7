// decode.hip -- one new query row per sequence against a prepped KV cache.
//
// softmax(q k^T scale) v over the first lens[b] cache rows (gizml:netops reference
// page, Functions > attention with tq = 1: the row sees the whole cache), with the
// query's HeadPrep (RMS, qw, split-half turn at table row pos[b]) applied as it is
// read.  The pass is HBM-bound: every cached key and value is read exactly once.
//
// Split-KV: a block owns one (sequence, kv head, group of up to 8 q heads, key split).
// The q heads of one kv head share every K/V read.  Its 4 waves take interleaved
// chunks of 16 keys and each keeps an online softmax (running max m, sum l, output
// a, rescaled by 2^(m_old - m_new) when m moves; scores are in base-2 units).
//   - Q K^T runs on the matrix cores with the chunk's keys as the 16 rows of A and
//     the (up to 8) prepped q heads as columns of B: v_mfma_f32_16x16x32_bf16 for
//     bf16 caches, v_mfma_f32_16x16x4f32 for f32 caches.  Each lane loads 16 bytes of
//     one key row straight into its A fragment.
//   - P V runs on the vector ALUs: d/8 (bf16) lanes share one value row, each lane
//     holding 8 of its values, and the chunk's weights come through LDS.
// The waves' states are merged in LDS and the block writes one partial (m, l, a[d])
// per q head to the workspace; a second kernel merges the splits (the same rescale
// applied across splits) and divides by l.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kChunk = 16;       // keys per wave step (the 16 rows of one MFMA)

struct DecodeParams {
    const void *q; const void *k; const void *v;
    float *work;
    int64_t batch, hq, hkv, capacity, max_len, per_split, splits;
    const int32_t *lens, *pos;
    const float *qw, *cos, *sin;
    int half, table_rows, group, ngroups;
    float eps, C;
    bool prep_q;
};

template <bool BF16, int D, int GB>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const DecodeParams p) {
    constexpr int ES = BF16 ? 2 : 4;          // bytes per element
    constexpr int VE = 16 / ES;               // elements per 16-byte load
    constexpr int LPK = D / VE;               // lanes per value row
    constexpr int KPI = 64 / LPK;             // value rows per wave load
    constexpr int KA = BF16 ? 8 : 4;          // A-fragment elements per lane per MFMA row-slot group
    constexpr int NKC = D / (4 * KA);         // 16-byte K loads per lane per chunk

    __shared__ float qs[GB][D];               // q rows, then normed
    __shared__ float qh[GB][D];               // prepped q
    __shared__ float pb[kWaves][kChunk][GB];  // chunk weights
    __shared__ float ab[kWaves][GB];          // chunk rescale factors
    __shared__ float wm[kWaves][GB], wl[kWaves][GB];
    __shared__ float wo[kWaves][GB][D];

    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64;
    const int split = blockIdx.x;
    const int kvh = blockIdx.y / p.ngroups, grp = blockIdx.y % p.ngroups;
    const int b = blockIdx.z;
    const int h0 = kvh * p.group + grp * GB;
    const int nh = min(GB, p.group - grp * GB);

    // Clamp what the device reads; the merge kernel turns bad lens/pos into NaN.
    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.max_len ? (int)p.max_len : len);
    const int start = split * (int)p.per_split;
    const int end = min(len, start + (int)p.per_split);

    // ---- q prologue (through LDS, any half).
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
        if (LPH > 64) {   // reduce across the waves of one head
            __shared__ float part[kThreads / 64];
            if (lane == 0) part[w] = ss;
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
            if (e < p.half) {
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

    // ---- B fragments: lane (n = lane % 16 head, kk = lane / 16).
    const int n = lane % 16, kk = lane / 16;
    typedef typename std::conditional<BF16, bf16x8, float>::type BFrag;
    BFrag qb[BF16 ? D / 32 : D / 4];
    if constexpr (BF16) {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (n < nh) {
                const float *src = &qh[n][32 * c + 8 * kk];
                u.x = pack_bf16x2(src[0], src[1]);
                u.y = pack_bf16x2(src[2], src[3]);
                u.z = pack_bf16x2(src[4], src[5]);
                u.w = pack_bf16x2(src[6], src[7]);
            }
            qb[c] = __builtin_bit_cast(bf16x8, u);
        }
    } else {
        // MFMA 4c + j takes d = 16c + 4kk + j (the order of a lane's 16-byte K load).
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) qb[4 * c + j] = n < nh ? qh[n][16 * c + 4 * kk + j] : 0.f;
    }

    const uint8_t *kbase = static_cast<const uint8_t *>(p.k) + (((int64_t)b * p.capacity) * p.hkv + kvh) * D * ES;
    const uint8_t *vbase = static_cast<const uint8_t *>(p.v) + (((int64_t)b * p.capacity) * p.hkv + kvh) * D * ES;
    const int64_t rowb = p.hkv * D * ES;      // bytes between consecutive cache rows

    float m_run = -INFINITY, l_run = 0.f;     // state of head n (replicated over kk)
    const int kq = lane / LPK, dseg = lane % LPK;
    float o[GB][VE];
#pragma unroll
    for (int i = 0; i < GB; ++i)
#pragma unroll
        for (int e = 0; e < VE; ++e) o[i][e] = 0.f;

    for (int key0 = start + kChunk * w; key0 < end; key0 += kChunk * kWaves) {
        // K rows -> A fragments; V rows -> registers.
        uint4 kr[NKC];
        const int kj = key0 + (lane % 16);
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
            // bf16: d = 32c + 8kk; f32: d = 16c + 4kk (16 bytes each)
            const int d0 = BF16 ? 32 * c + 8 * kk : 16 * c + 4 * kk;
            kr[c] = kj < end ? *reinterpret_cast<const uint4 *>(kbase + kj * rowb + d0 * ES) : make_uint4(0, 0, 0, 0);
        }
        uint4 vr[kChunk / KPI];
#pragma unroll
        for (int i = 0; i < kChunk / KPI; ++i) {
            const int vj = key0 + KPI * i + kq;
            vr[i] = vj < end ? *reinterpret_cast<const uint4 *>(vbase + vj * rowb + dseg * 16) : make_uint4(0, 0, 0, 0);
        }

        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF16) {
#pragma unroll
            for (int c = 0; c < NKC; ++c)
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[c]), qb[c], s, 0, 0, 0);
        } else {
#pragma unroll
            for (int c = 0; c < NKC; ++c) {
                const float kv[4] = {__uint_as_float(kr[c].x), __uint_as_float(kr[c].y),
                                     __uint_as_float(kr[c].z), __uint_as_float(kr[c].w)};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    s = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[j], qb[4 * c + j], s, 0, 0, 0);
            }
        }
        // lane (n, kk) holds keys key0 + 4kk + i, i < 4, for head n.
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = key0 + 4 * kk + i < end ? s[i] * p.C : -INFINITY;
            mx = fmaxf(mx, s[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);          // finite: key0 < end
        const float alpha = fast_exp2(m_run - m_new);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = fast_exp2(s[i] - m_new);
            ps += s[i];
        }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l_run = l_run * alpha + ps;
        m_run = m_new;
        if (n < GB) {
#pragma unroll
            for (int i = 0; i < 4; ++i) pb[w][4 * kk + i][n] = s[i];
            if (kk == 0) ab[w][n] = alpha;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

        float al[GB];
#pragma unroll
        for (int i = 0; i < GB; ++i) al[i] = ab[w][i];
#pragma unroll
        for (int i = 0; i < GB; ++i)
#pragma unroll
            for (int e = 0; e < VE; ++e) o[i][e] *= al[i];
#pragma unroll
        for (int r = 0; r < kChunk / KPI; ++r) {
            float vv[VE];
            if constexpr (BF16) {
                unpack_bf16x2(vr[r].x, vv[0], vv[1]);
                unpack_bf16x2(vr[r].y, vv[2], vv[3]);
                unpack_bf16x2(vr[r].z, vv[4], vv[5]);
                unpack_bf16x2(vr[r].w, vv[6], vv[7]);
            } else {
                vv[0] = __uint_as_float(vr[r].x); vv[1] = __uint_as_float(vr[r].y);
                vv[2] = __uint_as_float(vr[r].z); vv[3] = __uint_as_float(vr[r].w);
            }
            const int key = KPI * r + kq;
#pragma unroll
            for (int i = 0; i < GB; ++i) {
                const float pw = pb[w][key][i];
#pragma unroll
                for (int e = 0; e < VE; ++e) o[i][e] = fmaf(pw, vv[e], o[i][e]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }

    // ---- merge the lanes that hold the same d (different keys), then the waves.
#pragma unroll
    for (int i = 0; i < GB; ++i)
#pragma unroll
        for (int e = 0; e < VE; ++e)
#pragma unroll
            for (int sh = LPK; sh < 64; sh <<= 1) o[i][e] += __shfl_xor(o[i][e], sh, 64);
    if (kq == 0) {
#pragma unroll
        for (int i = 0; i < GB; ++i)
#pragma unroll
            for (int e = 0; e < VE; ++e) wo[w][i][dseg * VE + e] = o[i][e];
    }
    if (n < GB && kk == 0) {
        wm[w][n] = m_run;
        wl[w][n] = l_run;
    }
    __syncthreads();
    const int64_t stride = (int64_t)D + 2;
    for (int idx = tid; idx < nh * D; idx += kThreads) {
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
        float *dst = p.work + ((int64_t)split * p.batch * p.hq + (int64_t)b * p.hq + h0 + i) * stride;
        dst[e] = A;
        if (e == 0) {
            dst[D] = M;
            dst[D + 1] = L;
        }
    }
}

// Merge the splits of one (sequence, q head) and write the output row.
template <bool BF16, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float *work, void *out, const int32_t *lens,
                                                         const int32_t *pos, int64_t batch, int64_t hq,
                                                         int64_t splits, int64_t max_len, int64_t table_rows,
                                                         bool check_pos) {
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / hq;
    const int e = threadIdx.x;
    const int64_t stride = (int64_t)D + 2;
    const int len = lens[b];
    bool bad = len < 0 || len > max_len;
    if (check_pos) {
        const int pr = pos[b];
        bad = bad || pr < 0 || pr >= table_rows;
    }
    float M = -INFINITY;
    for (int64_t s = 0; s < splits; ++s) M = fmaxf(M, work[(s * batch * hq + bh) * stride + D]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
        for (int64_t s = 0; s < splits; ++s) {
            const float *src = work + (s * batch * hq + bh) * stride;
            const float f = fast_exp2(src[D] - M);
            L += src[D + 1] * f;
            A += src[e] * f;
        }
    }
    float y = L > 0.f ? A / L : 0.f;
    if (bad) y = __builtin_nanf("");
    if constexpr (BF16) {
        f32x2 v2 = {y, 0.f};
        bf16x2 hv = __builtin_convertvector(v2, bf16x2);
        static_cast<uint16_t *>(out)[bh * D + e] = (uint16_t)(__builtin_bit_cast(uint32_t, hv) & 0xFFFFu);
    } else {
        static_cast<float *>(out)[bh * D + e] = y;
    }
}

template <bool BF16, int D, int GB>
void launch_split(const DecodeParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)p.splits, (unsigned)(p.hkv * p.ngroups), (unsigned)p.batch);
    hipLaunchKernelGGL((decode_split_kernel<BF16, D, GB>), grid, dim3(kThreads), 0, stream, p);
}

template <bool BF16, int D>
void launch_split_gb(const DecodeParams &p, int gb, hipStream_t stream) {
    switch (gb) {
        case 1: launch_split<BF16, D, 1>(p, stream); break;
        case 2: launch_split<BF16, D, 2>(p, stream); break;
        case 4: launch_split<BF16, D, 4>(p, stream); break;
        default: launch_split<BF16, D, 8>(p, stream); break;
    }
}

}  // namespace

int64_t decode_heads_per_block(int64_t hq, int64_t hkv) {
    const int64_t group = hq / hkv;
    int64_t gb = 1;
    while (gb < group && gb < 8) gb <<= 1;
    return gb;
}

int64_t decode_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t max_len) {
    const int64_t gb = decode_heads_per_block(hq, hkv);
    const int64_t groups = (hq / hkv + gb - 1) / gb;
    const int64_t units = batch * hkv * groups;
    int64_t splits = (1024 + units - 1) / units;                   // about 4 blocks per CU
    const int64_t most = (max_len + 255) / 256;                    // at least 256 keys each
    if (splits > most) splits = most;
    if (splits < 1) splits = 1;
    return splits;
}

size_t decode_workspace_bytes(int64_t batch, int64_t hq, int64_t d, int64_t splits) {
    return (size_t)splits * (size_t)batch * (size_t)hq * (size_t)(d + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream) {
    DecodeParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.work = a.work;
    p.batch = a.batch; p.hq = a.hq; p.hkv = a.hkv; p.capacity = a.capacity; p.max_len = a.max_len;
    p.splits = a.splits;
    const int64_t per = (a.max_len + a.splits - 1) / a.splits;
    p.per_split = (per + 63) / 64 * 64;
    p.lens = a.lens; p.pos = a.pos;
    p.qw = a.qw; p.cos = a.cos; p.sin = a.sin;
    p.half = a.prep_q ? (int)a.half : 0;
    p.table_rows = a.prep_q && a.half > 0 ? (int)a.table_rows : 1;
    p.group = (int)(a.hq / a.hkv);
    const int gb = (int)decode_heads_per_block(a.hq, a.hkv);
    p.ngroups = (p.group + gb - 1) / gb;
    p.eps = a.eps;
    p.C = a.scale * kLog2e;
    p.prep_q = a.prep_q;
    if (a.d == 64) {
        if (a.bf16) launch_split_gb<true, 64>(p, gb, stream); else launch_split_gb<false, 64>(p, gb, stream);
    } else {
        if (a.bf16) launch_split_gb<true, 128>(p, gb, stream); else launch_split_gb<false, 128>(p, gb, stream);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const bool check_pos = a.prep_q && a.half > 0;
    const dim3 grid((unsigned)(a.batch * a.hq));
    if (a.d == 64) {
        if (a.bf16)
            hipLaunchKernelGGL((decode_merge_kernel<true, 64>), grid, dim3(64), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, a.table_rows, check_pos);
        else
            hipLaunchKernelGGL((decode_merge_kernel<false, 64>), grid, dim3(64), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, a.table_rows, check_pos);
    } else {
        if (a.bf16)
            hipLaunchKernelGGL((decode_merge_kernel<true, 128>), grid, dim3(128), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, a.table_rows, check_pos);
        else
            hipLaunchKernelGGL((decode_merge_kernel<false, 128>), grid, dim3(128), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, a.table_rows, check_pos);
    }
    return hipGetLastError();
}

}  // namespace attn
