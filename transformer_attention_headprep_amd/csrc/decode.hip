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
#include <mutex>

#include "decode_common.h"

namespace attn {
namespace {

// At d = 128 at most two waves per SIMD are asked for: a higher hint caps the vector
// registers at 128 and the excess goes through accumulation registers inside the loop.
template <int D, int GB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : (GB <= 4 ? 4 : 3)))) void decode_bf16_kernel(const DecodeParams p) {
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
            r.k[i] = __builtin_amdgcn_raw_buffer_load_b128(seq_rsrc(kbase + crow * rowb + skip, bytes - skip), loff, 0, kStream);
            r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(seq_rsrc(vbase + crow * rowb + skip, bytes - skip), loff, 0, kStream);
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
// bf16 caches, whole cache rows per block (decode_rows_kernel).
//
// A block owns one (sequence, group of hb consecutive kv heads, key split), hb D = 512
// (or every kv head when there are fewer): wave w takes kv head hb0 + w and its q heads.
// Each chunk of 16 cache rows is the group's 1 KB piece of 16 rows of K (and of V) -- a
// page holds a multiple of 16 rows -- and moves to LDS by buffer loads that write LDS
// directly, 1 KB (one row piece) each, spread over the waves: memory sees contiguous
// kilobytes requested together, which streams faster than blocks that read each kv head's
// 2 D bytes of every row.  In LDS a chunk keeps the cache's layout [row][kv head][D]
// except that the 16-byte pieces of each head's row sit at the swizzled slots kslot /
// vslot (each lane of a load fetches the piece that belongs at its slot, so every load
// still covers contiguous cache bytes); a wave then reads its head's K and V fragments
// exactly as decode_bf16_kernel does, with the row pitch hb 2 D.  A ring of four chunk
// buffers keeps three chunks in flight while one is computed, one barrier a chunk.
// Every wave holds the whole online-softmax state of its heads, so it writes its partial
// (or, with one split, its output rows) itself.
// Order one wave's LDS writes before its later reads of what other lanes wrote.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int GB>
__global__ __launch_bounds__(512) void decode_rows_kernel(const DecodeParams p, const int hb) {
    typedef DecGeo<D> G;
    // four chunk buffers of 2 kChunk hb 2 D <= 32 KB bytes (K then V): separate variables,
    // so the compiler sees that reads of one never depend on loads into another
    constexpr int kSlot = 2 * kChunk * 1024;
    constexpr int kDepth = 3;                        // chunks in flight while one is computed
    __shared__ __attribute__((aligned(16))) unsigned char cb0[kSlot];
    __shared__ __attribute__((aligned(16))) unsigned char cb1[kSlot];
    __shared__ __attribute__((aligned(16))) unsigned char cb2[kSlot];
    __shared__ __attribute__((aligned(16))) unsigned char cb3[kSlot];
    __shared__ float qst[8 * 512];                  // q staging: hb GB D <= 8 x 512 floats

    const int lane = threadIdx.x % 64;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int nw = hb;                               // waves = kv heads of the block
    const int RPb = nw * G::kRow;                    // LDS row pitch: the group's piece of a row
    const int64_t RP = p.hkv * G::kRow;              // cache row pitch
    const int split = (int)blockIdx.y, b = (int)blockIdx.z;
    const int kvh = (int)blockIdx.x * nw + w;
    const int h0 = kvh * p.group;
    const int nh = p.group;                          // <= GB

    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.max_len ? (int)p.max_len : len);
    const int start = split * (int)p.per_split;
    const int end = min(len, start + (int)p.per_split);
    const int nch = end > start ? (end - start + kChunk - 1) / kChunk : 0;   // block-uniform

    // ---- the loads of a chunk: K is 16 RPb bytes = 16 RPb / 1024 loads of 1 KB, V the
    // same; wave w issues loads w, w + nw, ... of each (D / 32 of each).  Lane L of load
    // i fills LDS bytes 1024 i + 16 L: row r, head h, slot c_pos; it fetches piece c_pos ^
    // swizzle(r) of that head's row from the cache.
    constexpr int per_w = D / 32;
    int64_t koff[per_w], voff[per_w];
#pragma unroll
    for (int x = 0; x < per_w; ++x) {
        const int off = 1024 * (w + nw * x) + 16 * lane;
        const int r = off / RPb, o = off - r * RPb;
        const int h = o / G::kRow, cpos = (o - h * G::kRow) / 16;
        koff[x] = r * RP + h * G::kRow + 16 * kslot<D>(r, cpos);
        voff[x] = r * RP + h * G::kRow + 16 * vslot<D>(r, cpos);
    }
    const int64_t urows = unit_rows(p);
    const int64_t hoff = (int64_t)blockIdx.x * nw * G::kRow;   // the group's first head in a row
    bool page_bad = false;
    // Chunk j into buf.  A chunk past the split (the first three are always issued) is an
    // empty range: its loads read nothing and write zeros.
    auto issue = [&](int j, unsigned char *buf) __attribute__((always_inline)) {
        const int key0 = start + kChunk * j;
        const bool some = key0 < end;
        const CacheSlot cs = some ? cache_slot(p, b, key0, page_bad) : CacheSlot{0, 0};
        const int64_t crow = (int64_t)cs.unit * urows + cs.row;
        // rows past the end read as zeros: the range ends with the last valid row's piece
        const int64_t bytes = some ? (int64_t)(min(kChunk, end - key0) - 1) * RP + RPb : 0;
        const __amdgpu_buffer_rsrc_t kr = seq_rsrc(static_cast<const uint8_t *>(p.k) + crow * RP + hoff, bytes);
        const __amdgpu_buffer_rsrc_t vr = seq_rsrc(static_cast<const uint8_t *>(p.v) + crow * RP + hoff, bytes);
#pragma unroll
        for (int x = 0; x < per_w; ++x) {
            // (the cache is read once: streamed, so it neither evicts nor waits behind
            // lines that other work left to be written back)
            buffer_to_lds16<kStream>(kr, buf + 1024 * (w + nw * x), (int)koff[x]);
            buffer_to_lds16<kStream>(vr, buf + kChunk * RPb + 1024 * (w + nw * x), (int)voff[x]);
        }
    };

    // ---- q prologue (per wave, its q heads).  q, the weights and the turn's cos / sin
    // are loaded into registers first, so that waiting for them later leaves the first
    // three chunks in flight: lane (head qi, part li) holds elements li EPL .. +EPL-1.
    constexpr int LPH = 64 / GB, EPL = D / LPH;
    const int qi = lane / LPH, li = lane % LPH;
    float xq[EPL], xw[EPL], xc[EPL], xs[EPL];
    // Every load is unconditional and in one basic block with the first chunks' issue
    // (absent inputs read a stand-in element of lens, clamped indices; the values are
    // selected after), so that they are all in flight together.
    const bool turn = p.prep_q && p.half > 0;
    const int pr = p.half > 0 ? p.pos[b] : 0;
    const int prow = pr < 0 ? 0 : (pr >= p.table_rows ? p.table_rows - 1 : pr);
    {
        const uint16_t *qrow = static_cast<const uint16_t *>(p.q) + ((int64_t)b * p.hq + h0 + min(qi, nh - 1)) * D + li * EPL;
        const float *qwp = p.prep_q ? p.qw + li * EPL : reinterpret_cast<const float *>(p.lens);
        const float *cp = turn ? p.cos + (int64_t)prow * p.half : reinterpret_cast<const float *>(p.lens);
        const float *sp = turn ? p.sin + (int64_t)prow * p.half : reinterpret_cast<const float *>(p.lens);
#pragma unroll
        for (int e0 = 0; e0 < EPL; ++e0) {
            const int e = li * EPL + e0;
            const int f = !turn ? 0 : (p.pairs ? min(e >> 1, p.half - 1) : (e < p.half ? e : min(e - p.half, p.half - 1)));
            xq[e0] = bf16_bits_to_f32(qrow[e0]);
            xw[e0] = qwp[p.prep_q ? e0 : 0];
            xc[e0] = cp[f];
            xs[e0] = sp[f];
        }
    }
    issue(0, cb0);
    issue(1, cb1);
    issue(2, cb2);
#pragma unroll
    for (int e0 = 0; e0 < EPL; ++e0) {
        const int e = li * EPL + e0;
        const bool turned = turn && (p.pairs ? (e >> 1) < p.half : e < 2 * p.half);
        if (qi >= nh) xq[e0] = 0.f;
        if (!p.prep_q) xw[e0] = 1.f;
        if (!turned) {
            xc[e0] = 1.f;
            xs[e0] = 0.f;
        }
    }

    // HeadPrep at table row pos[b] through this wave's rows of qst, then the B fragments
    // of S^T in registers: lane (head n, kk) holds q[n][32c + 8kk .. +7] as a bf16 high
    // part and a bf16 remainder (about 16 bits of q).
    float (*qs)[D] = reinterpret_cast<float (*)[D]>(qst + w * GB * D);
    const int n = lane % 16, kk = lane / 16;
    u32x4 qhi[G::kKMfma], qlo[G::kKMfma];
    {
        if (p.prep_q) {
            // head qi's sum of squares by its LPH lanes, then x qw / rms
            float ss = 0.f;
#pragma unroll
            for (int e0 = 0; e0 < EPL; ++e0) ss += xq[e0] * xq[e0];
            ss = sum_lanes<LPH>(ss);
            const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / D) + p.eps);
#pragma unroll
            for (int e0 = 0; e0 < EPL; ++e0) xq[e0] = xq[e0] * inv * xw[e0];
        }
#pragma unroll
        for (int e0 = 0; e0 < EPL; ++e0) qs[qi][li * EPL + e0] = xq[e0];
        wave_lds_sync();
        if (p.prep_q && p.half > 0) {
            // the turn: each element with its partner (the neighbour in the pair, or the
            // element half a table row away), read back from LDS
#pragma unroll
            for (int e0 = 0; e0 < EPL; ++e0) {
                const int e = li * EPL + e0;
                const float c = xc[e0], sn = xs[e0];
                float y = xq[e0];
                if (p.pairs) {
                    if ((e >> 1) < p.half) y = (e & 1) ? xq[e0] * c + qs[qi][e - 1] * sn : xq[e0] * c - qs[qi][e + 1] * sn;
                } else if (e < p.half) {
                    y = xq[e0] * c - qs[qi][e + p.half] * sn;
                } else if (e < 2 * p.half) {
                    y = xq[e0] * c + qs[qi][e - p.half] * sn;
                }
                xc[e0] = y;
            }
            wave_lds_sync();
#pragma unroll
            for (int e0 = 0; e0 < EPL; ++e0) qs[qi][li * EPL + e0] = xc[e0];
            wave_lds_sync();
        }
#pragma unroll
        for (int c = 0; c < G::kKMfma; ++c) {
            qhi[c] = u32x4{0u, 0u, 0u, 0u};
            qlo[c] = u32x4{0u, 0u, 0u, 0u};
            if (n < nh) {
                const float *src = &qs[n][32 * c + 8 * kk];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = src[2 * e], b2 = src[2 * e + 1];
                    qhi[c][e] = pack_bf16x2(a, b2);
                    float ha, hb;
                    unpack_bf16x2(qhi[c][e], ha, hb);
                    qlo[c][e] = pack_bf16x2(a - ha, b2 - hb);
                }
            }
        }
    }

    f32x4 acc[G::kNT];
#pragma unroll
    for (int t = 0; t < G::kNT; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, thr = -INFINITY, l_lane = 0.f;
    const int vkey = 4 * kk + (lane % 16) / 4, qq = lane % 4;

    auto compute = [&](int j, const unsigned char *buf) __attribute__((always_inline)) {
        const int key0 = start + kChunk * j;
        const unsigned char *kb = buf + w * G::kRow;
        const unsigned char *vb = buf + kChunk * RPb + w * G::kRow;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < G::kKMfma; c += 2) {
            bf16x8 kc[2];
            lds_read_b128_x2(kc[0], kc[1], lds_offset(kb + n * RPb + 16 * kslot<D>(n, 4 * c + kk)),
                             lds_offset(kb + n * RPb + 16 * kslot<D>(n, 4 * c + 4 + kk)));
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[u], __builtin_bit_cast(bf16x8, qhi[c + u]), s, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[u], __builtin_bit_cast(bf16x8, qlo[c + u]), s, 0, 0, 0);
            }
        }
        if (key0 + kChunk > end) {            // ragged last chunk (wave-uniform)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (key0 + 4 * kk + i >= end) s[i] = -INFINITY;
        }
        const float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
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
        const unsigned char *vrow = vb + vkey * RPb + 8 * (qq % 2);
#pragma unroll
        for (int t0 = 0; t0 < G::kNT; t0 += 4) {
            i16x4 a[4];
            lds_read_tr16_x4(a[0], a[1], a[2], a[3], lds_offset(vrow + 16 * vslot<D>(vkey, 2 * t0 + qq / 2)),
                             lds_offset(vrow + 16 * vslot<D>(vkey, 2 * t0 + 2 + qq / 2)),
                             lds_offset(vrow + 16 * vslot<D>(vkey, 2 * t0 + 4 + qq / 2)),
                             lds_offset(vrow + 16 * vslot<D>(vkey, 2 * t0 + 6 + qq / 2)));
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc[t0 + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[u], pf, acc[t0 + u], 0, 0, 0);
        }
    };
    // Chunk j: wait until this wave's loads of it are in (the two younger chunks may
    // still fly), a barrier publishes every wave's loads and ends every wave's reads of
    // chunk j-1, chunk j+3 goes into chunk j-1's buffer, chunk j is computed.  Unrolled by
    // four so each buffer is named at compile time.
    auto step = [&](int j, const unsigned char *cur, unsigned char *nextd) __attribute__((always_inline)) {
        const int younger = min(kDepth - 1, max(nch, kDepth) - 1 - j);   // chunks issued after chunk j
        if (younger >= 2) {
            ATTN_WAIT_VMCNT(4 * per_w);
        } else if (younger == 1) {
            ATTN_WAIT_VMCNT(2 * per_w);
        } else {
            ATTN_WAIT_VMCNT(0);
        }
        lds_barrier();
        if (j + kDepth < nch) issue(j + kDepth, nextd);
        compute(j, cur);
    };
    for (int j = 0; j < nch; j += 4) {
        step(j, cb0, cb3);
        if (j + 1 >= nch) break;
        step(j + 1, cb1, cb0);
        if (j + 2 >= nch) break;
        step(j + 2, cb2, cb1);
        if (j + 3 >= nch) break;
        step(j + 3, cb3, cb2);
    }
    ATTN_WAIT_VMCNT(0);       // empty chunks past a short split write LDS too

    // ---- this wave's heads: l over the head's 4 lanes, then the partial or the output.
    float l_head = l_lane + __shfl_xor(l_lane, 16, 64);
    l_head += __shfl_xor(l_head, 32, 64);
    if (n < nh) {
        const int64_t row = (int64_t)b * p.hq + h0 + n;
        const int64_t stride = (int64_t)D + 2;
        if (p.direct) {
            bool bad = page_bad;
            const int lr = p.lens[b];
            bad = bad || lr < 0 || lr > p.max_len;
            if (p.check_pos) {
                const int pp = p.pos[b];
                bad = bad || pp < 0 || pp >= p.table_rows;
            }
            const float inv = l_head > 0.f ? 1.0f / l_head : 0.f;
            const uint32_t nan_mask = bad ? 0xFFFFFFFFu : 0u;
            uint16_t *orow = static_cast<uint16_t *>(p.out) + row * D;
#pragma unroll
            for (int t = 0; t < G::kNT; ++t) {
                uint2 u;
                u.x = pack_bf16x2(acc[t][0] * inv, acc[t][1] * inv);
                u.y = pack_bf16x2(acc[t][2] * inv, acc[t][3] * inv);
                u.x = (u.x & ~nan_mask) | (0x7FC07FC0u & nan_mask);
                u.y = (u.y & ~nan_mask) | (0x7FC07FC0u & nan_mask);
                *reinterpret_cast<uint2 *>(orow + 16 * t + 4 * kk) = u;
            }
        } else {
            float *dst = p.work + ((int64_t)split * p.batch * p.hq + row) * stride;
#pragma unroll
            for (int t = 0; t < G::kNT; ++t) *reinterpret_cast<f32x4 *>(dst + 16 * t + 4 * kk) = acc[t];
            if (kk == 0) {
                dst[D] = m_run;
                dst[D + 1] = page_bad ? __builtin_nanf("") : l_head;   // the merge turns a NaN sum into NaN rows
            }
        }
    }
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

// Output elements lane + 64 e of row bh: A / L, NaN for a bad row or a NaN sum.
template <bool BF16, int D>
__device__ __forceinline__ void merge_store(void *out, int64_t bh, int lane, const float (&A)[D / 64], float L, bool bad) {
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
        float y = L > 0.f ? A[e] / L : 0.f;
        if (bad || L != L) y = __builtin_nanf("");
        if constexpr (BF16) {
            f32x2 v2 = {y, 0.f};
            bf16x2 hv = __builtin_convertvector(v2, bf16x2);
            static_cast<uint16_t *>(out)[bh * D + lane + 64 * e] = (uint16_t)(__builtin_bit_cast(uint32_t, hv) & 0xFFFFu);
        } else {
            static_cast<float *>(out)[bh * D + lane + 64 * e] = y;
        }
    }
}

// Merge the splits of one (sequence, q head) and write the output row: one wave a row.
// Lane s holds split s's maximum and sum (splits beyond 64 are read again in later
// passes); the split weights 2^(m_s - M) are computed once, by their lane, and read by
// every lane for its D / 64 output elements.
template <bool BF16, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float *work, void *out, const int32_t *lens,
                                                          const int32_t *pos, int64_t batch, int64_t hq,
                                                          int64_t splits, int64_t max_len, int64_t table_rows,
                                                          bool check_pos) {
    constexpr int EPL = D / 64;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / hq;
    const int lane = threadIdx.x;
    const int64_t stride = (int64_t)D + 2;
    const int64_t sstride = batch * hq * stride;     // from one split's rows to the next's
    const float *base = work + bh * stride;
    const int len = lens[b];
    bool bad = len < 0 || len > max_len;
    if (check_pos) {
        const int pr = pos[b];
        bad = bad || pr < 0 || pr >= table_rows;
    }
    if (splits <= 8) {
        // up to 8 splits: every load at once (indices clamped, values masked after), then
        // the sums in split order
        float m[8], l[8], v[8][EPL];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float *src = base + (s < splits ? s : splits - 1) * sstride;
            m[s] = src[D];
            l[s] = src[D + 1];
#pragma unroll
            for (int e = 0; e < EPL; ++e) v[s][e] = src[lane + 64 * e];
        }
        float M = -INFINITY;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            if (s < splits) M = fmaxf(M, m[s]);
        float L = 0.f, A[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) A[e] = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                if (s < splits) {
                    const float f = fast_exp2(m[s] - M);
                    L += l[s] * f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) A[e] += v[s][e] * f;
                }
            }
        }
        merge_store<BF16, D>(out, bh, lane, A, L, bad);
        return;
    }
    float m0 = -INFINITY, l0 = 0.f;
    if (lane < splits) {
        m0 = base[lane * sstride + D];
        l0 = base[lane * sstride + D + 1];
    }
    float M = m0;
    for (int64_t s = lane + 64; s < splits; s += 64) M = fmaxf(M, base[s * sstride + D]);
    M = max_lanes<64>(M);
    float A[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) A[e] = 0.f;
    float L = 0.f;
    if (M != -INFINITY) {
        for (int64_t s0 = 0; s0 < splits; s0 += 64) {
            const int64_t s = s0 + lane;
            float m = m0, l = l0;
            if (s0 > 0) {
                m = s < splits ? base[s * sstride + D] : -INFINITY;
                l = s < splits ? base[s * sstride + D + 1] : 0.f;
            }
            const float f = s < splits ? fast_exp2(m - M) : 0.f;
            L += l * f;
            const int n = (int)(splits - s0 < 64 ? splits - s0 : 64);
            const float *src = base + s0 * sstride + lane;
#pragma unroll 4
            for (int i = 0; i < n; ++i) {
                const float fi = __shfl(f, i, 64);
#pragma unroll
                for (int e = 0; e < EPL; ++e) A[e] += src[i * sstride + 64 * e] * fi;
            }
        }
        L = sum_lanes<64>(L);
    }
    merge_store<BF16, D>(out, bh, lane, A, L, bad);
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

// Launch of decode_rows_kernel: grid (splits, kv-head groups, batch), a wave per kv head
// of a group of hb D = 512 (or all hkv when fewer).
int decode_rows_group(int64_t hkv, int64_t d) {
    int hb = (int)(512 / d);
    while (hb > 1 && hkv % hb != 0) hb >>= 1;
    return hb < (int)hkv ? hb : (int)hkv;
}

template <int D, int GB>
hipError_t launch_rows(const DecodeLaunch &a, const DecodeParams &p, hipStream_t stream) {
    const int hb = decode_rows_group(a.hkv, D);
    hipLaunchKernelGGL((decode_rows_kernel<D, GB>), dim3((unsigned)(a.hkv / hb), (unsigned)a.splits, (unsigned)a.batch),
                       dim3((unsigned)(64 * hb)), 0, stream, p, hb);
    return hipGetLastError();
}

}  // namespace

int64_t decode_heads_per_block(int64_t hq, int64_t hkv) {
    const int64_t group = hq / hkv;
    int64_t gb = 1;
    while (gb < group && gb < 8) gb <<= 1;
    return gb;
}

bool decode_rows_fits(int64_t hq, int64_t hkv) {
    return hkv <= 8 && hq / hkv <= 8;      // a wave per kv head, up to 8 q heads each
}

int64_t decode_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t d, int64_t max_len) {
    if (decode_rows_fits(hq, hkv)) {
        // a block per (sequence, group of kv heads, split): about one block per CU (one
        // round of blocks), at least 256 keys each
        const int64_t groups = hkv / decode_rows_group(hkv, d);
        int64_t splits = (kCUs + batch * groups - 1) / (batch * groups);
        const int64_t most = (max_len + 255) / 256;
        if (splits > most) splits = most;
        return splits < 1 ? 1 : splits;
    }
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
    // About one round of blocks: a second round pays the q prologue again.  The kernel's
    // registers leave two blocks resident per CU with 8-bit keys and three with 4- or 2-bit
    // keys (measured at d = 128: 8/8 fastest at two blocks a CU, 4/4 and 4/2 at three).
    const int64_t gb = decode_heads_per_block(hq, hkv);
    const int64_t units = batch * hkv * ((hq / hkv + gb - 1) / gb);
    const int64_t blocks = (kbits == 8 ? 2 : 3) * kCUs;
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

// The split partials of attn_decode_static: a fixed array in device memory instead of a
// caller's workspace.  Every device the library runs on holds its own copy, at its own
// address, until the process ends.  Host code uses only the address that
// hipGetSymbolAddress returns for the current device (the array's name in host code is
// a host-side stand-in, not a device address).
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
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
            hipLaunchKernelGGL((decode_merge_kernel<true, 128>), grid, dim3(64), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, table_rows, check_pos);
        else
            hipLaunchKernelGGL((decode_merge_kernel<false, 128>), grid, dim3(64), 0, stream, a.work, a.out, a.lens, a.pos, a.batch, a.hq, a.splits, a.max_len, table_rows, check_pos);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream) {
    if (a.kbits) return launch_decode_q(a, stream);
    const DecodeParams p = make_decode_params(a);
    const int gb = (int)decode_heads_per_block(a.hq, a.hkv);
    if (a.bf16 && decode_rows_fits(a.hq, a.hkv)) {
        hipError_t err = hipSuccess;
        if (a.d == 64) {
            switch (gb) {
                case 1: err = launch_rows<64, 1>(a, p, stream); break;
                case 2: err = launch_rows<64, 2>(a, p, stream); break;
                case 4: err = launch_rows<64, 4>(a, p, stream); break;
                default: err = launch_rows<64, 8>(a, p, stream); break;
            }
        } else {
            switch (gb) {
                case 1: err = launch_rows<128, 1>(a, p, stream); break;
                case 2: err = launch_rows<128, 2>(a, p, stream); break;
                case 4: err = launch_rows<128, 4>(a, p, stream); break;
                default: err = launch_rows<128, 8>(a, p, stream); break;
            }
        }
        if (err != hipSuccess) return err;
        return launch_decode_merge(a, stream);
    }
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
