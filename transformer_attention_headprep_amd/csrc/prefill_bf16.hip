// prefill_bf16.hip -- bf16 attention of whole sequences on the gfx950 matrix cores.
//
// softmax(q k^T scale [+ causal mask]) v (gizml:netops reference page, Functions >
// attention) with the (tq, tk) scores never leaving the chip: keys go in tiles of 64
// through LDS, and each query row keeps a running maximum, sum and output that are
// rescaled when the maximum moves (the online softmax described there and on the
// gpukit page's fused attention).  Products run on v_mfma_f32_32x32x16_bf16 with f32
// accumulation; the output is rounded to bf16 once at the end.
//
// Work split: a block of 4 waves owns 128 query rows of one (batch, q head); each
// wave owns 32 rows.  Both products are computed transposed so that one lane always
// holds one query row:
//   S^T = K Q^T   (A = K tile from LDS, B = prepped Q held in registers)
//   O^T += V^T P^T (A = V^T read from LDS with ds_read_b64_tr_b16, B = P straight
//                   from the S^T accumulator registers)
// With that layout the row maximum is a max over a lane's own 32 scores plus one
// exchange with lane ^ 32 (v_permlane32_swap), and the rescale of O needs no exchange.
//
// Tiles move HBM -> LDS by buffer loads that write LDS directly (no registers, no LDS
// store instructions), double-buffered: tile kt+1 is in flight while tile kt is used,
// one barrier per tile.  The two buffers are two LDS variables and the tile loop is
// unrolled by two, so each read names its buffer at compile time: the compiler then
// knows that a read of one buffer does not depend on the loads still writing the other,
// and inserts no wait for them (with one buffer array indexed at run time, every
// transposing V read waited for the next tile's loads).  A step issues the next tile's
// loads after its K reads: issued at the top of the step, they made the first unrolled
// copy's K reads wait for them (the compiler's wait insertion loses the two buffers
// apart where the loop's state merges), which left that copy with no overlap at all.
// K fragments are read from LDS two 16-wide chunks ahead of the products that take them.
// The buffer descriptor of a tile ends with the sequence, so keys past its end arrive as
// zeros.  K rows are stored 16 bytes wider than their data and V rows 64 bytes wider (the
// extra slots are filled by the same loads): K row pitches step 4 banks, so the 16-byte
// reads of 16 consecutive key rows cover all 64 banks once; V row pitches step 16 banks,
// so the transposing reads of 4 key rows x 64 bytes by 32 lanes do too.  Every LDS offset is then an immediate.  Two blocks fit a
// CU (2 waves per SIMD).
//
// The ds_read_b64_tr_b16 layout (gfx950): in each group of 16 lanes, lane i receives
// element (i mod 4) of the 4-element vectors addressed by lanes 4r + i/4, r = 0..3.
// So lanes 4r .. 4r+3 address 4 consecutive values of key row r, and every lane
// receives one column (one d) across 4 keys: the A fragment of V^T.
//
// Online softmax in base-2 units.  A prepped q (computed in f32 anyway) is multiplied
// by scale log2 e before it is rounded to bf16, and every S^T accumulation starts from
// -m (the row's running maximum, held in 16 registers), so the matrix core returns
// s log2 e - m directly and the weights are a bare v_exp_f32 of the accumulator.  A q
// given without HeadPrep is used as it is (rescaling it would round it a second time)
// and the exponent takes one multiply by scale log2 e instead.  The running maximum is
// only raised when a tile's maximum exceeds it by more than 8 (base 2): the weights
// 2^(s - m) then stay below 256, which f32 sums and bf16 weights hold exactly as well
// as weights below 1, and the rescale of O (64 multiplies a lane) is skipped on almost
// every tile.  The result is the same softmax: numerator and denominator use the same
// m.  The row sum adds the bf16-rounded weights that the P V product uses
// (v_dot2_f32_bf16), so numerator and denominator match.
//
// Fixed shift: with q's HeadPrep fused and a bound kb on the norm of every key row
// (the caller's kmax, or sqrt(D) max|kw| when the call prepped k from kw), no score of
// query row n exceeds |q_n| kb (Cauchy-Schwarz, on the bf16 values the matrix cores
// take).  A wave whose rows all have |q_n| kb <= 48 starts every row at m = |q_n| kb and
// keeps no running maximum: the same softmax (any shift no score exceeds gives it), with
// every weight in [2^-96, 1], and no max, exchange or raise test per tile.
//
// The q prologue applies HeadPrep (RMS, qw, split-half turn at the row's position)
// in registers before rounding q to bf16; it needs half to be 0 or a multiple of 16
// (then every turned pair sits in one lane).  Other halves are prepped by the prep
// kernel beforehand.
//
// Block order: longest causal query tiles first; when the (batch, kv head) pairs
// divide evenly over the 8 XCDs, every pair's blocks go to one XCD (blocks are
// dealt to XCDs round-robin), so its K/V stay in that XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn {

hipError_t launch_prefill_f32(const PrefillLaunch &a, hipStream_t stream);

namespace {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;   // query rows per block
constexpr int kBN = 64;            // keys per tile
constexpr int kXcds = 8;
constexpr float kRaiseAbove = 8.0f;   // base-2 headroom before the running max moves
constexpr float kFixedShiftMax = 48.0f;   // largest fixed softmax shift (base 2) a row may take

__shared__ int prefill_bad_page;      // a K/V page id outside the pool was met

// The value held by lane ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float lane_pair(float x, int g) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(g == 0 ? r[1] : r[0]);
}

// Split-half turn of a lane's q values held as NC chunks of 8 (chunk c = d 16c + 8g ..):
// chunk c < HC pairs with chunk c + HC (half = 16 HC); cv / sv hold the table entries
// 16c + 8g .. + 7 of the row for each c < HC.
template <int NC, int HC>
__device__ __forceinline__ void turn_chunks(float (&x)[NC][8], const f32x4 (&cv)[NC / 2][2],
                                            const f32x4 (&sv)[NC / 2][2]) {
    if constexpr (HC >= 1 && 2 * HC <= NC) {
#pragma unroll
        for (int c = 0; c < HC; ++c) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float co = cv[c][e / 4][e % 4], si = sv[c][e / 4][e % 4];
                const float a = x[c][e], b = x[c + HC][e];
                x[c][e] = a * co - b * si;
                x[c + HC][e] = b * co + a * si;
            }
        }
    }
}

// How a launch's grid carries the block coordinates (see launch_bf16_d): the query tile
// is z (reversed: longest causal tiles first); the (batch, kv head) pair and the q head
// within its kv group sit on x and y, so a block finds them with no division but one
// multiply-shift by hkv.
struct PrefillGrid {
    int mode;          // 0: x = 8 group (x % 8 = pair % 8, x / 8 = head in group), y = pair / 8
                       // 1: x = head in group, y = pair;  2: x = pair, y = head in group
    int group;         // q heads per kv head
    int hkv;
    uint32_t hkv_mul;  // pair / hkv = (pair hkv_mul) >> hkv_shift for 0 <= pair < 2^31
    int hkv_shift;
};

// LDS geometry of one tile buffer for head dim D.
template <int D>
struct Geo {
    static constexpr int kRow = 2 * D;                   // data bytes of one key row
    static constexpr int kChunks = D / 8;                // 16-byte chunks of data per row
    static constexpr int kKStride = kRow + 16;           // K row pitch (one pad slot)
    static constexpr int kVStride = kRow + 64;           // V row pitch (four pad slots)
    static constexpr int kKSlots = kKStride / 16;
    static constexpr int kVSlots = kVStride / 16;
    static constexpr int kKBytes = kBN * kKStride;
    static constexpr int kVBytes = kBN * kVStride;
    static constexpr int kBufBytes = kKBytes + kVBytes;
    static constexpr int kKLoads = kBN * kKSlots / 64;   // 64-lane loads per K tile
    static constexpr int kVLoads = kBN * kVSlots / 64;
    static constexpr int kPerWave = (kVLoads + 1) / 2;   // waves 0,1 load K; 2,3 load V
    static_assert(kBN * kKSlots % 64 == 0 && kBN * kVSlots % 64 == 0, "whole 64-lane loads");
};

template <int D, bool CAUSAL, bool PREP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_bf16_kernel(const PrefillLaunch p,
                                                                                                    const PrefillGrid gr) {
    typedef Geo<D> G;
    // The two tile buffers are separate variables so that the compiler sees that reads of
    // one never wait for the loads in flight into the other.
    __shared__ __attribute__((aligned(16))) unsigned char tb0[G::kBufBytes];
    __shared__ __attribute__((aligned(16))) unsigned char tb1[G::kBufBytes];
    constexpr int NC = D / 16;       // 16-wide d chunks of the q.k product
    constexpr int NDB = D / 32;      // 32-wide d blocks of the output

    const int lane = threadIdx.x % 64;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);   // wave-uniform: scalar addressing
    const int n = lane % 32, g = lane / 32;

    // ---- which (batch, q head, query tile) this block owns
    const int tq = (int)p.seq, tk = (int)p.tk, qoff = tk - tq;   // query i sits at key position i + qoff
    const int qtile = (int)gridDim.z - 1 - (int)blockIdx.z;
    int pair, hg;
    if (gr.mode == 0) {
        pair = (int)(blockIdx.x % kXcds) + kXcds * (int)blockIdx.y;
        hg = (int)(blockIdx.x / kXcds);
    } else if (gr.mode == 1) {
        pair = (int)blockIdx.y;
        hg = (int)blockIdx.x;
    } else {
        pair = (int)blockIdx.x;
        hg = (int)blockIdx.y;
    }
    const int b = (int)(((uint64_t)(uint32_t)pair * gr.hkv_mul) >> gr.hkv_shift);
    const int kvh = pair - b * gr.hkv;
    const int h = kvh * gr.group + hg;

    const int64_t row0w = (int64_t)qtile * kBM + 32 * w;           // first row of this wave
    const int wrows = (int)max<int64_t>(0, min<int64_t>(32, tq - row0w));   // its rows inside the sequence
    const int64_t r = row0w + n;
    const bool row_ok = r < tq;

    const int64_t last_key = CAUSAL ? min<int64_t>(tk - 1, (int64_t)qtile * kBM + kBM - 1 + qoff) : tk - 1;
    const int ntiles = (int)(last_key / kBN) + 1;

    // ---- tile loads: waves 0 and 1 move K, waves 2 and 3 move V; load t of a wave
    // fills 64 consecutive 16-byte slots; a slot past a row's data repeats its last
    // chunk (it is padding, never read).
    const bool loads_k = w < 2;
    const int wl = w & 1;
    const int nloads = loads_k ? (G::kKLoads - wl + 1) / 2 : (G::kVLoads - wl + 1) / 2;
    const int64_t rs = loads_k ? p.k_rs : p.v_rs;
    const bool paged = p.kv_pages.pages != nullptr;
    const uint16_t *src = static_cast<const uint16_t *>(loads_k ? p.k : p.v) +
                          (paged ? 0 : (int64_t)b * (loads_k ? p.k_bs : p.v_bs)) + (int64_t)kvh * D;
    bool bad_page = false;
    int voff[G::kPerWave];
#pragma unroll
    for (int t = 0; t < G::kPerWave; ++t) {
        const int sidx = (wl + 2 * t) * 64 + lane;
        const int row = loads_k ? sidx / G::kKSlots : sidx / G::kVSlots;   // constant divisors
        const int col = sidx - row * (loads_k ? G::kKSlots : G::kVSlots);
        voff[t] = (int)(row * rs + 8 * min(col, G::kChunks - 1)) * 2;
    }
    // A paged pool holds a 64-key tile in one page (pages are a power of two >= 64 rows).
    auto load_tile = [&](int kt, unsigned char *tbuf) {
        const int key0 = kt * kBN;
        __amdgpu_buffer_rsrc_t rsrc;
        if (paged) {
            const int64_t prow = pool_row(p.kv_pages, b, key0, bad_page);
            rsrc = seq_rsrc(src + prow * rs, ((int64_t)(min(kBN, tk - key0) - 1) * rs + D) * 2);
        } else {
            rsrc = seq_rsrc(src + (int64_t)key0 * rs, ((int64_t)(tk - 1 - key0) * rs + D) * 2);
        }
        unsigned char *dst = tbuf + (loads_k ? 0 : G::kKBytes);
#pragma unroll
        for (int t = 0; t < G::kPerWave; ++t) {
            if (t < nloads)
                buffer_to_lds16(rsrc, dst + (wl + 2 * t) * 1024, voff[t]);
        }
    };

    // First tile on its way before the q prologue.
    if (threadIdx.x == 0) prefill_bad_page = 0;      // read only after the loop's barriers
    load_tile(0, tb0);

    const float C = p.scale * kLog2e;       // q is scaled by this before it is rounded

    // ---- q prologue: this lane's 64 (or 32) values of its row, HeadPrep, bf16.  Every
    // load is issued before anything waits; rows past the sequence (and table rows past
    // them) read as zeros through the wave's descriptors.
    bf16x8 qf[NC];
    float kb = 0.f;        // PREP: bound on the norm of every key row (0: none known)
    float shift = 0.f;     // |q| kb, a bound on every score of the row
    {
        const __amdgpu_buffer_rsrc_t qsrc =
            seq_rsrc(static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_bs + row0w * p.q_rs + (int64_t)h * D,
                     wrows > 0 ? ((int64_t)(wrows - 1) * p.q_rs + D) * 2 : 0);
        const int qoff_lane = (n * (int)p.q_rs + 8 * g) * 2;
        u32x4 raw[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) raw[c] = __builtin_amdgcn_raw_buffer_load_b128(qsrc, qoff_lane + 32 * c, 0, 0);
        if constexpr (PREP) {
            const int hc = (int)p.half / 16;     // turned pairs are hc chunks apart
            f32x4 wv[NC][2], cv[NC / 2][2], sv[NC / 2][2];
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int j = 0; j < 2; ++j) wv[c][j] = *reinterpret_cast<const f32x4 *>(p.qw + 16 * c + 8 * g + 4 * j);
            if (hc > 0) {
                const int64_t tbytes = (int64_t)wrows * p.half * 4;
                const __amdgpu_buffer_rsrc_t crs = seq_rsrc(p.cos + (p.pos0 + row0w) * p.half, tbytes);
                const __amdgpu_buffer_rsrc_t srs = seq_rsrc(p.sin + (p.pos0 + row0w) * p.half, tbytes);
                const int toff = (n * (int)p.half + 8 * g) * 4;
#pragma unroll
                for (int c = 0; c < NC / 2; ++c)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        if (c < hc) {
                            cv[c][j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, toff + 64 * c + 16 * j, 0, 0));
                            sv[c][j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, toff + 64 * c + 16 * j, 0, 0));
                        }
            }
            // Sum of squares straight from the bf16 pairs (exact products, f32 sums).
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bf16x8 v8 = __builtin_bit_cast(bf16x8, raw[c]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x2 pr = {v8[2 * j], v8[2 * j + 1]};
                    ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
                }
            }
            ss += __shfl_xor(ss, 32, 64);
            // x qw, turned, then one multiply by the row's 1 / rms and scale log2 e (both
            // steps are linear, so the order is the method's up to rounding).
            float x[NC][8];
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float lo, hi;
                    unpack_bf16x2(raw[c][j], lo, hi);
                    x[c][2 * j] = lo * wv[c][j / 2][(2 * j) % 4];
                    x[c][2 * j + 1] = hi * wv[c][j / 2][(2 * j + 1) % 4];
                }
            // hc is a run-time value; dispatch to unrolled code so x stays in registers.
            switch (hc) {
                case 0: break;
                case 1: turn_chunks<NC, 1>(x, cv, sv); break;
                case 2: turn_chunks<NC, 2>(x, cv, sv); break;
                case 3: turn_chunks<NC, 3>(x, cv, sv); break;
                default: turn_chunks<NC, NC / 2>(x, cv, sv); break;
            }
            const float f = C * __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                uint4 u;
                u.x = pack_bf16x2(x[c][0] * f, x[c][1] * f);
                u.y = pack_bf16x2(x[c][2] * f, x[c][3] * f);
                u.z = pack_bf16x2(x[c][4] * f, x[c][5] * f);
                u.w = pack_bf16x2(x[c][6] * f, x[c][7] * f);
                qf[c] = __builtin_bit_cast(bf16x8, u);
            }
            // Key-norm bound: the caller's kmax, and when this call prepped k from kw,
            // sqrt(D) max|kw| (each prepped key row is its RMS-normed values times kw,
            // turned, rounded to bf16) -- whichever is smaller.
            kb = p.kmax;
            if (p.kwb) {
                float a = fabsf(p.kwb[lane % D]);
                if constexpr (D > 64) a = fmaxf(a, fabsf(p.kwb[64 + lane % (D - 64)]));
                const float kw_bound = __builtin_sqrtf((float)D) * max_lanes<64>(a) * (1.0f + 1.0f / 128);
                kb = kb > 0.f ? fminf(kb, kw_bound) : kw_bound;
            }
            if (kb > 0.f) {
                // |q| of the bf16 values the products take; Cauchy-Schwarz bounds each
                // score by |q| kb, and the margin covers the f32 accumulation.
                float qn = 0.f;
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bf16x2 pr = {qf[c][2 * j], qf[c][2 * j + 1]};
                        qn = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, qn, false);
                    }
                qn += __shfl_xor(qn, 32, 64);
                shift = __builtin_sqrtf(qn) * kb * (1.0f + 1.0f / 1024);
            }
        } else {
            // q is taken as given: scaling it before the product would round it twice.
#pragma unroll
            for (int c = 0; c < NC; ++c) qf[c] = __builtin_bit_cast(bf16x8, raw[c]);
        }
    }
    // Accumulator units: base 2 when q carries scale log2 e (PREP), else raw q.k, which
    // the exponent then scales.
    const float sc = PREP ? 1.0f : C;
    // Fixed shift: when every row of the wave has a score bound no larger than
    // kFixedShiftMax, each row's softmax is shifted by its bound from the start (the
    // same softmax: numerator and denominator share the shift; every weight lies in
    // [2^-96, 1], where f32 and bf16 keep their relative precision) and no running
    // maximum is kept.  Otherwise the running maximum below.
    const bool fixed = PREP && kb > 0.f &&
                       __builtin_amdgcn_ballot_w64(!(shift <= kFixedShiftMax)) == 0;   // wave-uniform
    float m_run = fixed ? shift : -INFINITY, l_run = 0.f;   // l_run: this lane's share of the row sum
    f32x16 bias;                             // -m_run (0 until the first visible key)
#pragma unroll
    for (int i = 0; i < 16; ++i) bias[i] = fixed ? -shift : 0.f;
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // Per-lane LDS byte offsets (the rest of every address is an immediate).
    const int k_lane = n * G::kKStride + 16 * g;                        // K row n, chunk g
    const int j16 = lane % 16, rg = (lane % 32) / 16;
    const int v_lane = G::kKBytes + (4 * g + j16 / 4) * G::kVStride + (16 * rg + 4 * (j16 % 4)) * 2;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Key positions of this wave's first and last row: a tile whose first key lies past the
    // last row's is skipped by the wave (it still loads and waits with the block).
    const int64_t wfirst = row0w + qoff, wlast = row0w + 31 + qoff;
    auto step = [&](int kt, const unsigned char *buf, unsigned char *next) __attribute__((always_inline)) {
        const int key0 = kt * kBN;
        if (wrows == 0 || (CAUSAL && key0 > wlast)) {
            if (kt + 1 < ntiles) load_tile(kt + 1, next);
            if (bad_page && lane == 0) prefill_bad_page = 1;   // seen by all after this tile's barrier
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            return;
        }

        // S^T = K Q^T - m for 2 blocks of 32 keys (two independent accumulation chains).
        f32x16 s[2];
        bf16x8 ka[NC][2];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                ka[c][kb] = *reinterpret_cast<const bf16x8 *>(buf + k_lane + kb * 32 * G::kKStride + 32 * c);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c][kb], qf[c], c == 0 ? bias : s[kb], 0, 0, 0);
        }
        // reads run two chunks ahead of the products
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * NC - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (kt + 1 < ntiles) load_tile(kt + 1, next);
        if (bad_page && lane == 0) prefill_bad_page = 1;   // seen by all after this tile's barrier
        // Mask: register 4i+jj of block kb holds key key0 + 32 kb + 8 i + 4 g + jj.
        const bool need_mask = (key0 + kBN > tk) || (CAUSAL && key0 + kBN - 1 > wfirst);
        if (need_mask) {
            const int lim = (CAUSAL ? min(tk - 1, (int)r + qoff) : tk - 1) - (key0 + 4 * g);   // last visible
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kb + 8 * (i / 4) + (i % 4) > lim) s[kb][i] = -INFINITY;
        }
        float mx = -INFINITY;
        if (!fixed) {
            mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
            for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[0][i], s[0][i + 1]));
#pragma unroll
            for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[1][i], s[1][i + 1]));
            mx = fmaxf(mx, lane_pair(mx, g));                 // tile max of s - m
        }
        const bool first = m_run == -INFINITY;
        const bool raise = !fixed && (first ? mx > -INFINITY : mx * sc > kRaiseAbove);
        if (__builtin_amdgcn_ballot_w64(raise)) {            // wave-uniform, rare
            const float delta = raise ? mx : 0.f;
            const float alpha = fast_exp2(-delta * sc);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            if (raise) m_run = (first ? 0.f : m_run) + delta;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] -= delta;
            const float nb = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
            for (int i = 0; i < 16; ++i) bias[i] = nb;
        }

        // P as the B operand: step u covers keys 16u..16u+15 (registers 8(u%2).. of block u/2),
        // slot s of lane half g holding key 16u + 8(s/4) + 4g + s%4.
        bf16x8 pf[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float e8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) e8[i] = fast_exp2(s[u / 2][8 * (u % 2) + i] * sc);
            uint4 pk;
            pk.x = pack_bf16x2(e8[0], e8[1]);
            pk.y = pack_bf16x2(e8[2], e8[3]);
            pk.z = pack_bf16x2(e8[4], e8[5]);
            pk.w = pack_bf16x2(e8[6], e8[7]);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk.x), ones, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk.y), ones, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk.z), ones, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk.w), ones, l_run, false);
            pf[u] = __builtin_bit_cast(bf16x8, pk);
        }
        // O^T += V^T P^T: the A fragment of (d block db, keys of step u) is two transposing
        // reads, keys 16u + 4g + 0..3 and 16u + 8 + 4g + 0..3 (the slot order of P).
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const unsigned char *va = buf + v_lane + 16 * u * G::kVStride + 64 * db;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(va));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(va + 8 * G::kVStride));
                const i16x4 both[2] = {lo, hi};
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pf[u], o[db], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);        // this wave's loads of tile kt+1 are in LDS
        __syncthreads();
    };
    for (int kt = 0; kt < ntiles; kt += 2) {
        step(kt, tb0, tb1);
        if (kt + 1 < ntiles) step(kt + 1, tb1, tb0);
    }

    // ---- epilogue: divide by the row sum, round once to bf16, store.
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (row_ok) {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        // A bad page: quiet-NaN bf16 bits (set as integers: this file is built without NaN semantics).
        const uint32_t nan_mask = prefill_bad_page ? 0xFFFFFFFFu : 0u;
        uint16_t *orow = static_cast<uint16_t *>(p.out) + (int64_t)b * p.o_bs + r * p.o_rs + (int64_t)h * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint2 u;
                u.x = pack_bf16x2(o[db][4 * i] * inv, o[db][4 * i + 1] * inv);
                u.y = pack_bf16x2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
                u.x = (u.x & ~nan_mask) | (0x7FC07FC0u & nan_mask);
                u.y = (u.y & ~nan_mask) | (0x7FC07FC0u & nan_mask);
                *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * i + 4 * g) = u;
            }
    }
}

// Grid: z = query tile; when the (batch, kv head) pairs divide evenly over the XCDs,
// x = 8 group so that consecutive blocks (dealt to XCDs round-robin) put each pair's
// blocks on one XCD; else x and y carry head-in-group and pair.  Launch order is x,
// then y, then z: the heads of one kv group run side by side, longest tiles first.
template <int D, bool CAUSAL>
hipError_t launch_bf16_d(const PrefillLaunch &a, hipStream_t stream) {
    const int64_t nq_tiles = (a.seq + kBM - 1) / kBM;
    const int64_t group = a.hq / a.hkv, pairs = a.batch * a.hkv;
    if (nq_tiles > 65535 || group > 65535 || pairs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    PrefillGrid gr;
    dim3 grid;
    if (pairs % kXcds == 0 && kXcds * group <= 65535 && pairs / kXcds <= 65535) {
        gr.mode = 0;
        grid = dim3((unsigned)(kXcds * group), (unsigned)(pairs / kXcds), (unsigned)nq_tiles);
    } else if (pairs <= 65535) {
        gr.mode = 1;
        grid = dim3((unsigned)group, (unsigned)pairs, (unsigned)nq_tiles);
    } else {
        gr.mode = 2;
        grid = dim3((unsigned)pairs, (unsigned)group, (unsigned)nq_tiles);
    }
    gr.group = (int)group;
    gr.hkv = (int)a.hkv;
    int l = 0;
    while (((int64_t)1 << l) < a.hkv) ++l;                    // ceil(log2 hkv)
    gr.hkv_mul = (uint32_t)((((uint64_t)1 << (31 + l)) + (uint64_t)a.hkv - 1) / (uint64_t)a.hkv);
    gr.hkv_shift = 31 + l;
    const size_t lds = 0;
    if (a.prep_q)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, true>), grid, dim3(256), lds, stream, a, gr);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, false>), grid, dim3(256), lds, stream, a, gr);
    return hipGetLastError();
}

}  // namespace

bool prefill_fuses_half(int64_t d, int64_t half, bool bf16) {
    if (!bf16) return half == 0 || 2 * half == d;
    return half == 0 || half % 16 == 0;   // pairs 1, 2, 3 or 4 chunks of 16 apart
}

void prefill_defaults(PrefillLaunch &a) {
    if (a.tk == 0) a.tk = a.seq;
    if (a.q_bs == 0) a.q_bs = a.seq * a.q_rs;
    if (a.o_bs == 0) a.o_bs = a.seq * a.o_rs;
    if (a.k_bs == 0) a.k_bs = a.tk * a.k_rs;
    if (a.v_bs == 0) a.v_bs = a.tk * a.v_rs;
}

hipError_t launch_prefill(const PrefillLaunch &a0, hipStream_t stream) {
    PrefillLaunch a = a0;
    prefill_defaults(a);
    if (!a.bf16) return launch_prefill_f32(a, stream);
    if (a.d == 64) return a.causal ? launch_bf16_d<64, true>(a, stream) : launch_bf16_d<64, false>(a, stream);
    return a.causal ? launch_bf16_d<128, true>(a, stream) : launch_bf16_d<128, false>(a, stream);
}

}  // namespace attn
