// decode.hip -- one new query row per sequence against a prepped KV cache.
//
// softmax(q k^T scale) v over the first lens[b] cache rows (gizml:netops reference
// page, Functions > attention with tq = 1: the row sees the whole cache), with the
// query's HeadPrep (RMS, qw, split-half turn at table row pos[b]) applied as it is
// read.  The pass is HBM-bound: every cached key and value is read exactly once.
//
// Split-KV: a block owns one (sequence, kv head, group of up to 8 q heads, key split).
// The q heads of one kv head share every K/V read.  Its 4 waves take interleaved
// chunks of 16 keys and each keeps an online softmax in base-2 units (running max m,
// sum l, output a).  The waves' states are merged in LDS and the block writes one
// partial (m, l, a[d]) per q head to the workspace; a second kernel merges the splits
// (the same rescale applied across splits) and divides by l.
//
// bf16 caches (decode_bf16_kernel): both products on the matrix cores.
//   - every load instruction reads whole cache rows of the kv head (4 rows of 256 bytes
//     for d = 128); a wave stores its chunk's 16 K rows and 16 V rows to swizzled LDS
//     buffers and reads them back in the layouts the matrix cores take.
//   - S^T = K Q^T with v_mfma_f32_16x16x32_bf16: the chunk's 16 keys are the rows of A,
//     the q heads the columns of B, once as bf16 and once as the bf16 remainder of the
//     prepped f32 q.  Lane (head n, kk) ends up with keys 4kk .. 4kk+3 of head n.
//   - O^T += V^T P^T with v_mfma_f32_16x16x16_bf16: those four probabilities, rounded to
//     bf16, are exactly the lane's B fragment; V^T fragments come from transposing LDS
//     reads (ds_read_b64_tr_b16).  No probability or value passes through the vector
//     ALUs.
//   - the running max only moves when a score exceeds it by more than 2^8 (a
//     wave-uniform branch); otherwise a chunk costs 4 exponentials per lane.
//   - the loads of chunk j+1 are in flight while chunk j is computed.
//   - each (sequence, kv head) starts at a hashed chunk of its range and wraps around, so
//     the blocks' streams do not move through equally spaced sequences in lockstep.
// f32 caches (decode_f32_kernel): S^T on v_mfma_f32_16x16x4f32, P V on the vector ALUs
// (D/4 lanes share one value row) with the chunk's weights passed through LDS.
#include "decode_common.h"

namespace attn {
namespace {

template <int D, int GB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(GB <= 4 ? 4 : 3))) void decode_bf16_kernel(const DecodeParams p) {
    typedef DecGeo<D> G;
    constexpr int kTiles = kWaves * 2 * G::kBuf;               // K and V chunk of every wave
    constexpr int kQBytes = 2 * GB * D * 4 + 4 * (kThreads / 64);
    constexpr int kOBytes = kWaves * GB * D * 4 + 2 * kWaves * GB * 4;
    static_assert(kQBytes <= kTiles && kOBytes <= kTiles, "prologue and merge fit the tile region");
    constexpr int kQFrag = 2 * G::kKMfma * 64 * 16;            // B fragments of S^T, read every chunk
    // One LDS region, reused: q rows (prologue), then one K and one V chunk per wave,
    // then the waves' outputs (after a block barrier); the q fragments follow it.
    __shared__ __attribute__((aligned(16))) unsigned char smem[kTiles + kQFrag];
    __shared__ int s_page_bad;                 // some wave met a page id outside the pool

    const int tid = threadIdx.x, lane = tid % 64;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    if (tid == 0) s_page_bad = 0;              // seen by all after the prologue's barriers
    const BlockCoord bc = block_coord(p);
    const int b = bc.b, split = bc.split;
    const int h0 = bc.kvh * p.group + bc.grp * GB;
    const int nh = min(GB, p.group - bc.grp * GB);

    // Clamp what the device reads; the merge kernel turns bad lens/pos into NaN.
    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.max_len ? (int)p.max_len : len);
    const int start = split * (int)p.per_split;
    const int end = min(len, start + (int)p.per_split);

    const int64_t rowb = p.hkv * D * 2;       // bytes between consecutive cache rows
    // Cache row r (of every sequence, or of the pool) starts at r rowb; this kv head's
    // part of it kvh D 2 bytes further.
    const uint8_t *kbase = static_cast<const uint8_t *>(p.k) + (int64_t)bc.kvh * D * 2;
    const uint8_t *vbase = static_cast<const uint8_t *>(p.v) + (int64_t)bc.kvh * D * 2;
    const int64_t urows = unit_rows(p);
    bool page_bad = false;
    unsigned char *kbuf = smem + w * 2 * G::kBuf;    // this wave's K chunk
    unsigned char *vbuf = kbuf + G::kBuf;            // and V chunk

    // Load i of a chunk: lane L reads 16 bytes (chunk L % kCpr) of row kRpi i + L / kCpr,
    // kRpi whole rows per instruction.  The row offset stays in the VGPR offset (the part
    // the descriptor's range check covers); each load has its own descriptor.
    const int lrow = lane / G::kCpr, lchunk = lane % G::kCpr;
    const int loff = lrow * (int)rowb + 16 * lchunk;

    // This wave's chunks: keys start + 16 (w + 4 j) .. +15, j < nch.
    const int first = start + kChunk * w;
    const int nch = end > first ? (end - first + kChunk * kWaves - 1) / (kChunk * kWaves) : 0;
    // Chunks are taken in a rotated order, starting at a chunk hashed from (sequence, kv
    // head): with every block starting at its first key, the blocks' streams sit at equal
    // offsets of equally spaced sequences and crowd the same memory channels.  The order
    // does not change the softmax (up to rounding); chunks past the last (j >= nch) keep
    // their place, past the end, so they fetch nothing.
    const int rot = nch > 0 ? (int)((((uint32_t)(b * (int)p.hkv + bc.kvh) * 2654435761u) >> 16) % (uint32_t)nch) : 0;
    auto chunk_of = [&](int j) { return j < nch ? (j + rot < nch ? j + rot : j + rot - nch) : j; };

    struct Regs {
        u32x4 k[G::kLoads];
        u32x4 v[G::kLoads];
    };
    // Chunk j's rows, read through descriptors that end at the cache's last valid row
    // (rows past it, and every row of a chunk past the end, read as zero without a fetch).
    // A chunk's 16 rows lie in one unit (pages hold a multiple of 16 rows).
    auto issue = [&](int j, Regs &r) {
        const int key0 = first + kChunk * kWaves * chunk_of(j);
        const int64_t bytes = (int64_t)min(kChunk, end - key0) * rowb;
        const CacheSlot cs = key0 < end ? cache_slot(p, b, key0, page_bad) : CacheSlot{0, 0};
        const int64_t crow = (int64_t)cs.unit * urows + cs.row;
#pragma unroll
        for (int i = 0; i < G::kLoads; ++i) {
            const int64_t skip = (int64_t)(G::kRpi * i) * rowb;
            r.k[i] = __builtin_amdgcn_raw_buffer_load_b128(seq_rsrc(kbase + crow * rowb + skip, bytes - skip), loff, 0, 0);
            r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(seq_rsrc(vbase + crow * rowb + skip, bytes - skip), loff, 0, 0);
        }
    };

    // The first chunk's rows are on their way (into registers) during the q prologue.
    Regs ra, rb;
    issue(0, ra);

    float (*qs)[D] = reinterpret_cast<float (*)[D]>(smem);
    float (*qh)[D] = reinterpret_cast<float (*)[D]>(smem + GB * D * 4);
    q_prologue<true, D, GB>(p, b, h0, nh, qs, qh, reinterpret_cast<float *>(smem + 2 * GB * D * 4));

    // B fragments of S^T: lane (head n, kk) holds q[n][32c + 8kk .. +7], split into a
    // bf16 high part and a bf16 remainder (q - high) so the scores carry q to about 16
    // bits rather than 8 (the matrix cores are idle enough to take both).  They are kept
    // in LDS (lane-linear, so reads are conflict-free) rather than in 32 VGPRs.
    const int n = lane % 16, kk = lane / 16;
    u32x4 *qf = reinterpret_cast<u32x4 *>(smem + kTiles);
    if (w == 0) {
#pragma unroll
        for (int c = 0; c < G::kKMfma; ++c) {
            u32x4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
            if (n < nh) {
                const float *src = &qh[n][32 * c + 8 * kk];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = src[2 * e], b2 = src[2 * e + 1];
                    hi[e] = pack_bf16x2(a, b2);
                    float ha, hb;
                    unpack_bf16x2(hi[e], ha, hb);
                    lo[e] = pack_bf16x2(a - ha, b2 - hb);
                }
            }
            qf[64 * (2 * c) + lane] = hi;
            qf[64 * (2 * c + 1) + lane] = lo;
        }
    }
    __syncthreads();     // q rows are dead: the LDS now holds K and V chunks

    f32x4 acc[G::kNT];
#pragma unroll
    for (int t = 0; t < G::kNT; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, thr = -INFINITY, l_lane = 0.f;

    // A wave's LDS operations run in order, so chunk j+1's stores cannot overtake
    // chunk j's reads of the same buffers.
    auto compute = [&](int j, const Regs &r) {
        const int key0 = first + kChunk * kWaves * chunk_of(j);
#pragma unroll
        for (int i = 0; i < G::kLoads; ++i) {
            const int row = G::kRpi * i + lrow;
            *reinterpret_cast<u32x4 *>(kbuf + row * G::kRow + 16 * kslot<D>(row, lchunk)) = r.k[i];
            *reinterpret_cast<u32x4 *>(vbuf + row * G::kRow + 16 * vslot<D>(row, lchunk)) = r.v[i];
        }
        // S^T: lane (key n, kk) takes chunk 4c + kk of its key row for MFMA c.
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < G::kKMfma; ++c) {
            const bf16x8 kc = *reinterpret_cast<const bf16x8 *>(kbuf + n * G::kRow + 16 * kslot<D>(n, 4 * c + kk));
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, __builtin_bit_cast(bf16x8, qf[64 * (2 * c) + lane]), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, __builtin_bit_cast(bf16x8, qf[64 * (2 * c + 1) + lane]), s, 0, 0, 0);
        }
        if (key0 + kChunk > end) {            // ragged last chunk (wave-uniform)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (key0 + 4 * kk + i >= end) s[i] = -INFINITY;
        }
        const float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
            // Raise the running max of every head to its max so far.
            float mh = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mh = fmaxf(mh, __shfl_xor(mh, 32, 64));
            const float m_new = fmaxf(m_run, mh * p.C);
            const float alpha = fast_exp2(m_run - m_new);
            l_lane *= alpha;
#pragma unroll
            for (int t = 0; t < G::kNT; ++t) acc[t] *= alpha;
            m_run = m_new;
            thr = (m_run + kRaiseAbove) / p.C;
        }
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(fmaf(s[i], p.C, -m_run));
        l_lane += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        const uint32_t p01 = pack_bf16x2(pr[0], pr[1]), p23 = pack_bf16x2(pr[2], pr[3]);
        const i16x4 pf = __builtin_bit_cast(i16x4, make_uint2(p01, p23));
        // O^T: for d tile t, lane 16g + 4r + q addresses V[4g + r][16t + 4q .. +3].
        const int vkey = 4 * kk + (lane % 16) / 4, q = lane % 4;
#pragma unroll
        for (int t = 0; t < G::kNT; ++t) {
            const i16x4 a = lds_read_tr16(vbuf + vkey * G::kRow + 16 * vslot<D>(vkey, 2 * t + q / 2) + 8 * (q % 2));
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pf, acc[t], 0, 0, 0);
        }
    };

    // Two chunks per iteration so the register buffers alternate statically;
    // chunk j+1 is in flight while chunk j is computed.  The chunk after the last one
    // is issued with empty descriptors (nothing fetched), which keeps the loop free of
    // branches around the loads.
    for (int j = 0; j < nch; j += 2) {
        issue(j + 1, rb);
        compute(j, ra);
        if (j + 1 >= nch) break;
        issue(j + 2, ra);
        compute(j + 1, rb);
    }

    // ---- merge: the lanes of one head (kk), then the waves.
    float l_head = l_lane + __shfl_xor(l_lane, 16, 64);
    l_head += __shfl_xor(l_head, 32, 64);
    if (page_bad && lane == 0) s_page_bad = 1;
    __syncthreads();                          // every wave is done with its chunk buffers
    float (*wo)[GB][D] = reinterpret_cast<float (*)[GB][D]>(smem);
    float (*wm)[GB] = reinterpret_cast<float (*)[GB]>(smem + kWaves * GB * D * 4);
    float (*wl)[GB] = reinterpret_cast<float (*)[GB]>(smem + kWaves * GB * D * 4 + kWaves * GB * 4);
    if (n < GB) {
#pragma unroll
        for (int t = 0; t < G::kNT; ++t) *reinterpret_cast<f32x4 *>(&wo[w][n][16 * t + 4 * kk]) = acc[t];
        if (kk == 0) {
            wm[w][n] = m_run;
            wl[w][n] = l_head;
        }
    }
    __syncthreads();
    write_partial<true, D, GB>(p, split, b, h0, nh, wm, wl, wo, s_page_bad != 0);
}

// ---------------------------------------------------------------------------------
// f32 caches.

template <int D, int GB>
__global__ __launch_bounds__(kThreads) void decode_f32_kernel(const DecodeParams p) {
    constexpr int VE = 4;                     // elements per 16-byte load
    constexpr int LPK = D / VE;               // lanes per value row
    constexpr int KPI = 64 / LPK;             // value rows per wave load
    constexpr int NKC = D / 16;               // 16-byte K loads per lane per chunk

    __shared__ float qs[GB][D];
    __shared__ float qh[GB][D];
    __shared__ float pb[kWaves][kChunk][GB];  // chunk weights
    __shared__ float ab[kWaves][GB];          // chunk rescale factors
    __shared__ float wm[kWaves][GB], wl[kWaves][GB];
    __shared__ float wo[kWaves][GB][D];

    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64;
    const BlockCoord bc = block_coord(p);
    const int b = bc.b, split = bc.split;
    const int h0 = bc.kvh * p.group + bc.grp * GB;
    const int nh = min(GB, p.group - bc.grp * GB);

    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.max_len ? (int)p.max_len : len);
    const int start = split * (int)p.per_split;
    const int end = min(len, start + (int)p.per_split);

    __shared__ float part[kThreads / 64];
    q_prologue<false, D, GB>(p, b, h0, nh, qs, qh, part);

    // B fragments: lane (n = lane % 16 head, kk = lane / 16); MFMA 4c + j takes
    // d = 16c + 4kk + j (the order of a lane's 16-byte K load).
    const int n = lane % 16, kk = lane / 16;
    float qb[D / 4];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) qb[4 * c + j] = n < nh ? qh[n][16 * c + 4 * kk + j] : 0.f;

    const uint8_t *kbase = static_cast<const uint8_t *>(p.k) + ((int64_t)b * p.capacity * p.hkv + bc.kvh) * D * 4;
    const uint8_t *vbase = static_cast<const uint8_t *>(p.v) + ((int64_t)b * p.capacity * p.hkv + bc.kvh) * D * 4;
    const int64_t rowb = p.hkv * D * 4;

    float m_run = -INFINITY, l_run = 0.f;     // state of head n (replicated over kk)
    const int kq = lane / LPK, dseg = lane % LPK;
    float o[GB][VE];
#pragma unroll
    for (int i = 0; i < GB; ++i)
#pragma unroll
        for (int e = 0; e < VE; ++e) o[i][e] = 0.f;

    for (int key0 = start + kChunk * w; key0 < end; key0 += kChunk * kWaves) {
        uint4 kr[NKC];
        const int kj = key0 + (lane % 16);
#pragma unroll
        for (int c = 0; c < NKC; ++c)
            kr[c] = kj < end ? *reinterpret_cast<const uint4 *>(kbase + kj * rowb + (16 * c + 4 * kk) * 4)
                             : make_uint4(0, 0, 0, 0);
        uint4 vr[kChunk / KPI];
#pragma unroll
        for (int i = 0; i < kChunk / KPI; ++i) {
            const int vj = key0 + KPI * i + kq;
            vr[i] = vj < end ? *reinterpret_cast<const uint4 *>(vbase + vj * rowb + dseg * 16) : make_uint4(0, 0, 0, 0);
        }

        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
            const float kv[4] = {__uint_as_float(kr[c].x), __uint_as_float(kr[c].y),
                                 __uint_as_float(kr[c].z), __uint_as_float(kr[c].w)};
#pragma unroll
            for (int j = 0; j < 4; ++j) s = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[j], qb[4 * c + j], s, 0, 0, 0);
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
            const float vv[VE] = {__uint_as_float(vr[r].x), __uint_as_float(vr[r].y), __uint_as_float(vr[r].z),
                                  __uint_as_float(vr[r].w)};
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
    write_partial<false, D, GB>(p, split, b, h0, nh, wm, wl, wo);
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
    if (bad || L != L) y = __builtin_nanf("");
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
    const dim3 grid((unsigned)(p.hkv * p.ngroups), (unsigned)p.splits, (unsigned)p.batch);
    if constexpr (BF16)
        hipLaunchKernelGGL((decode_bf16_kernel<D, GB>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_f32_kernel<D, GB>), grid, dim3(kThreads), 0, stream, p);
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
    if (units >= kCUs) return 1;                                   // a block per CU already
    int64_t splits = (4 * kCUs + units - 1) / units;               // about 4 blocks per CU
    const int64_t most = (max_len + 255) / 256;                    // at least 256 keys each
    if (splits > most) splits = most;
    if (splits < 1) splits = 1;
    return splits;
}

int64_t decode_q_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t max_len, int64_t kbits) {
    // A chunk of coded rows carries 2 (8 bits) to 4 (4 and 2 bits) times fewer bytes than a
    // bf16 one, so more blocks are needed to keep as many bytes in flight.
    const int64_t gb = decode_heads_per_block(hq, hkv);
    const int64_t units = batch * hkv * ((hq / hkv + gb - 1) / gb);
    const int64_t blocks = (kbits == 8 ? 2 : 4) * kCUs;
    int64_t splits = (blocks + units - 1) / units;
    const int64_t most = (max_len + 255) / 256;
    if (splits > most) splits = most;
    if (splits < 1) splits = 1;
    return splits;
}

size_t decode_workspace_bytes(int64_t batch, int64_t hq, int64_t d, int64_t splits) {
    if (splits <= 1) return 0;                                     // one split writes the output
    return (size_t)splits * (size_t)batch * (size_t)hq * (size_t)(d + 2) * sizeof(float);
}

DecodeParams make_decode_params(const DecodeLaunch &a) {
    DecodeParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.work = a.work; p.out = a.out;
    p.direct = a.splits == 1;
    p.check_pos = a.prep_q && a.half > 0;
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
    p.pairs = a.prep_q && a.pairs;
    p.kpar = a.kpar; p.vpar = a.vpar;
    p.pages = a.pages;
    p.page_shift = 0;
    if (a.pages)
        while (((int64_t)1 << p.page_shift) < a.page_rows) ++p.page_shift;
    p.max_pages = (int)a.max_pages;
    p.num_pages = (int)a.num_pages;
    return p;
}

hipError_t launch_decode_merge(const DecodeLaunch &a, hipStream_t stream) {
    if (a.splits <= 1) return hipSuccess;
    const bool check_pos = a.prep_q && a.half > 0;
    const int64_t table_rows = check_pos ? a.table_rows : 1;
    const dim3 grid((unsigned)(a.batch * a.hq));
    if (a.d == 64) {
        if (a.bf16)
            hipLaunchKernelGGL((decode_merge_kernel<true, 64>), grid, dim3(64), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, table_rows, check_pos);
        else
            hipLaunchKernelGGL((decode_merge_kernel<false, 64>), grid, dim3(64), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, table_rows, check_pos);
    } else {
        if (a.bf16)
            hipLaunchKernelGGL((decode_merge_kernel<true, 128>), grid, dim3(128), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, table_rows, check_pos);
        else
            hipLaunchKernelGGL((decode_merge_kernel<false, 128>), grid, dim3(128), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, table_rows, check_pos);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream) {
    if (a.kbits) return launch_decode_q(a, stream);
    const DecodeParams p = make_decode_params(a);
    const int gb = (int)decode_heads_per_block(a.hq, a.hkv);
    if (a.d == 64) {
        if (a.bf16) launch_split_gb<true, 64>(p, gb, stream); else launch_split_gb<false, 64>(p, gb, stream);
    } else {
        if (a.bf16) launch_split_gb<true, 128>(p, gb, stream); else launch_split_gb<false, 128>(p, gb, stream);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_decode_merge(a, stream);
}

}  // namespace attn
