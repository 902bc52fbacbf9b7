// prefill_bf16.hip -- bf16 attention of whole sequences: persistent blocks of two wave
// groups that take turns on the matrix cores.
//
// softmax(q k^T scale [+ causal mask]) v (gizml:netops reference page, Functions >
// attention), online softmax over 64-key tiles in LDS, products on
// v_mfma_f32_32x32x16_bf16 with f32 accumulation, the output rounded to bf16 once.
//
// A block has 8 waves in two groups of 4 (A = waves 0-3, B = waves 4-7); one block per
// CU, so every SIMD holds one wave of each group.  A work item is two query slots of
// 128 rows that read the same keys: two q heads of one kv head at the same query tile
// (an even number of q heads per kv head), or two consecutive query tiles of one q head
// (otherwise).  Group A takes the first slot, group B the second; each wave owns 32
// query rows and computes both products transposed so one lane holds one query row:
//   S^T = K Q^T    (A operand: K tile from LDS, B operand: prepped q in registers)
//   O^T += V^T P^T (A operand: V^T from LDS by ds_read_b64_tr_b16, B operand: P built
//                   from the S^T accumulators)
//
// Ping-pong: the two groups run the same tile sequence half a tile apart.  Each tile
// period has two phases separated by a block barrier; in every phase one group issues
// its matrix products -- Q K^T of tile t and P V of tile t-1, 32 MFMAs a wave at d 128
// -- while the other turns the scores of its previous tile into weights (exponentials,
// bf16 conversion, row sums: vector ALU work).  So on every SIMD one wave keeps the
// matrix core busy while the other uses the vector ALU, and the roles swap at each
// barrier.  The wave in its matrix phase raises its issue priority (s_setprio) so the
// other wave's vector work fills the gaps and never delays an MFMA.
//
//   phase 2t   : A: S(t) = K_t Q^T ; O += P(t-1) V_{t-1}     B: P(t-1) = exp(S(t-1))
//   phase 2t+1 : A: P(t) = exp(S(t))                        B: S(t), O += P(t-1) V_{t-1}
//
// K and V tiles move HBM -> LDS by buffer loads that write LDS directly, in rings of
// three buffers each (tile t in buffer t mod 3).  Group A's waves load K, group B's load
// V, each as its softmax phase starts (tile t + 2 then), so the loads never hold up a
// matrix phase; each tile has about a period and a half to arrive (see the tile steps
// below).  Row pitches are padded (K by 16 bytes, V by 64) so the 16-byte K fragment
// reads and the transposing V reads are free of bank conflicts with immediate offsets.
// A tile's buffer descriptor ends with the sequence: keys past it read as zeros.
//
// Work order: blocks are persistent (one per CU) and walk a static list.  When the
// (batch, kv head) pairs divide over the 8 XCDs, each pair's items go to the blocks of
// one XCD (blocks are dealt to XCDs round-robin), so its K/V stay in that XCD's L2.
// Within an XCD the items are sorted longest causal extent first and dealt to its
// blocks in a snake (block j takes items j, 2n-1-j, 2n+j, ... of n blocks), which evens
// the causal work per block.
//
// Online softmax in base-2 units: a prepped q is multiplied by scale log2 e before its
// bf16 rounding, so a score accumulator is already in base 2.  With a bound on every key
// row's norm (the caller's kmax, or sqrt(D) max|kw| when the call prepped k) and every
// row's bound |q_n| kb at most 48 (Cauchy-Schwarz: no score of row n exceeds it), the
// weights are bare exponentials of the accumulators and no maximum is kept; otherwise
// the running maximum moves only when a tile exceeds it by more than 8 (weights below
// 256, exact in f32 sums and bf16).  The row sum adds the f32 weights (the P V product
// takes their bf16 roundings).
//
// Between items: with two q heads a block (the slots share their query rows) the two
// groups run their prologues side by side and split the rotary table rows between them;
// those rows come by whole-row loads into LDS and are read back in the fragment layout,
// and each item's q loads are issued in the previous item's epilogue.  The output tile
// goes through LDS too, so that every store writes whole rows.
//
// q's HeadPrep (RMS, qw, split-half turn at the row's position, scale log2 e) runs in
// each wave's prologue in registers; it needs half = 0 or a multiple of 16.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn {

hipError_t launch_prefill_f32(const PrefillLaunch &a, hipStream_t stream);

namespace {

constexpr int kBN = 64;              // keys per tile
constexpr int kBM = 128;             // query rows per slot (4 waves x 32)
constexpr float kRaiseAbove = 8.0f;  // base-2 headroom before the running maximum moves
constexpr float kFixedShiftMax = 48.0f;

// The value held by lane ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float pp_lane_pair(float x, int g) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(g == 0 ? r[1] : r[0]);
}

// x unchanged, computed here: the compiler can neither hoist it out of a loop nor sink it
// (a value kept in a vector register, pp_pin_v, or a scalar one, pp_pin_s).
__device__ __forceinline__ int pp_pin_v(int x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ int pp_pin_s(int x) {
    asm volatile("" : "+s"(x));
    return x;
}

// 16 bytes per lane from a buffer straight into LDS (lane L writes lds + 16 L), at
// per-lane offset voff plus the wave-uniform soff.
__device__ __forceinline__ void pp_to_lds16(__amdgpu_buffer_rsrc_t rsrc, void *lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// Wait until at most k (0 .. 10) vector-memory operations of this wave are in flight
// (k is wave-uniform; the count is an immediate, hence the cases).
__device__ __forceinline__ void wait_vmcnt_upto(int k) {
    switch (k) {
        case 10: ATTN_WAIT_VMCNT(10); break;
        case 9: ATTN_WAIT_VMCNT(9); break;
        case 8: ATTN_WAIT_VMCNT(8); break;
        case 7: ATTN_WAIT_VMCNT(7); break;
        case 6: ATTN_WAIT_VMCNT(6); break;
        case 5: ATTN_WAIT_VMCNT(5); break;
        case 4: ATTN_WAIT_VMCNT(4); break;
        case 3: ATTN_WAIT_VMCNT(3); break;
        case 2: ATTN_WAIT_VMCNT(2); break;
        case 1: ATTN_WAIT_VMCNT(1); break;
        default: ATTN_WAIT_VMCNT(0); break;
    }
}

template <int D>
struct PPGeo {
    static constexpr int kRow = 2 * D;
    static constexpr int kChunks = D / 8;
    static constexpr int kKStride = kRow + 16;
    static constexpr int kVStride = kRow + 64;
    static constexpr int kKSlots = kKStride / 16;
    static constexpr int kVSlots = kVStride / 16;
    static constexpr int kKBytes = kBN * kKStride;
    static constexpr int kVBytes = kBN * kVStride;
    static constexpr int kKLoads = kBN * kKSlots / 64;   // 64-lane loads per K tile
    static constexpr int kVLoads = kBN * kVSlots / 64;
    static constexpr int kKPer = (kKLoads + 3) / 4;      // per loading wave (4 waves each)
    static constexpr int kVPer = (kVLoads + 3) / 4;
    static constexpr int kPer = kKPer > kVPer ? kKPer : kVPer;
};

// The launch's arguments, compact (row strides fit 32 bits: the ABI bounds them by 2^24).
struct PPArgs {
    const uint16_t *q, *k, *v;
    uint16_t *out;
    const float *qw, *cos, *sin, *kwb;
    int64_t q_bs, k_bs, v_bs, o_bs;
    int q_rs, k_rs, v_rs, o_rs;
    PageMap kv_pages;  // pages != NULL: k and v are paged pools (a 64-key tile lies in one page)
    const int32_t *past;  // != NULL: per-sequence cache lengths (PrefillLaunch::past)
    int tq, tk, half, pos0;
    float eps, scale, kmax;
    // items (see launch_bf16_d)
    int mode;          // 0: slots = q heads 2s, 2s+1 of a kv group at one query tile
                       // 1: slots = query tiles 2j, 2j+1 of one q head
    int group;         // q heads per kv head
    int hkv;
    int nsub;          // items per (pair, length class): group / 2 (mode 0) or group (mode 1)
    int nlen;          // length classes: query tiles (mode 0) or tile pairs (mode 1)
    int xcds;          // 8: pair p's items on XCD p % 8;  1: one list
    int ppx;           // pairs per list
    int nbx;           // blocks per list
    int items_x;       // items per list = nlen * ppx * nsub
};

// q's HeadPrep for one lane: raw holds the lane's NC chunks of 8 bf16 values of its row
// (chunk c = d 16c + 8g ..); chunk c < HC turns with chunk c + HC (half = 16 HC) by the
// row's cos/sin (cv, sv: chunk c's 8 values, loaded by the caller), from 2 HC on the
// values pass through.  Each pair of chunks is finished (weight, turn, the
// row's factor f = scale log2 e / rms, bf16) before the next one's weights are read, so
// no whole-row f32 copy is held.
template <int NC, int HC>
__device__ __forceinline__ void pp_prep_q(const u32x4 (&raw)[NC], const float *qw_lds, const f32x4 (&cv)[4][2],
                                          const f32x4 (&sv)[4][2], int g, float f, bf16x8 (&qf)[NC]) {
    auto weight = [&](int c, float (&x)[8]) __attribute__((always_inline)) {
        const f32x4 w0 = *reinterpret_cast<const f32x4 *>(qw_lds + 16 * c + 8 * g);
        const f32x4 w1 = *reinterpret_cast<const f32x4 *>(qw_lds + 16 * c + 8 * g + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float lo, hi;
            unpack_bf16x2(raw[c][j], lo, hi);
            x[2 * j] = lo * (j < 2 ? w0 : w1)[(2 * j) % 4];
            x[2 * j + 1] = hi * (j < 2 ? w0 : w1)[(2 * j + 1) % 4];
        }
    };
    auto pack = [&](const float (&x)[8]) __attribute__((always_inline)) {
        uint4 u;
        u.x = pack_bf16x2(x[0] * f, x[1] * f);
        u.y = pack_bf16x2(x[2] * f, x[3] * f);
        u.z = pack_bf16x2(x[4] * f, x[5] * f);
        u.w = pack_bf16x2(x[6] * f, x[7] * f);
        return __builtin_bit_cast(bf16x8, u);
    };
    if constexpr (HC >= 1 && 2 * HC <= NC) {
#pragma unroll
        for (int c = 0; c < HC; ++c) {
            float a[8], b[8];
            weight(c, a);
            weight(c + HC, b);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float co = cv[c][e / 4][e % 4], si = sv[c][e / 4][e % 4];
                const float x0 = a[e], x1 = b[e];
                a[e] = x0 * co - x1 * si;
                b[e] = x1 * co + x0 * si;
            }
            qf[c] = pack(a);
            qf[c + HC] = pack(b);
        }
    }
    constexpr int first_plain = (HC >= 1 && 2 * HC <= NC) ? 2 * HC : 0;
#pragma unroll
    for (int c = first_plain; c < NC; ++c) {
        float a[8];
        weight(c, a);
        qf[c] = pack(a);
    }
}

template <int D, bool CAUSAL, bool PREP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_bf16_kernel(const PPArgs p) {
    typedef PPGeo<D> G;
    // Separate variables per ring slot: the compiler then knows a read of one never
    // depends on loads in flight into another.
    __shared__ __attribute__((aligned(16))) unsigned char kb0[G::kKBytes];
    __shared__ __attribute__((aligned(16))) unsigned char kb1[G::kKBytes];
    __shared__ __attribute__((aligned(16))) unsigned char kb2[G::kKBytes];
    __shared__ __attribute__((aligned(16))) unsigned char vb0[G::kVBytes];
    __shared__ __attribute__((aligned(16))) unsigned char vb1[G::kVBytes];
    __shared__ __attribute__((aligned(16))) unsigned char vb2[G::kVBytes];
    __shared__ __attribute__((aligned(16))) float qw_s[D];
    // Rotary table staging of the prologue (see the prologue step): per wave, 32 rows of
    // cos then 32 of sin, each row KC 16-byte slots.  Waves 0, 1 of a group use tst, waves
    // 2, 3 the third K and V ring buffers.
    constexpr int KC = D / 8;                     // 16-byte chunks per q row
    constexpr int RPI = 64 / KC;                  // table rows per 64-lane load
    constexpr int NT = 32 / RPI;                  // loads per table
    constexpr int NV = KC / RPI > 1 ? KC / RPI : 1;   // swizzle patterns over the loads
    constexpr int kTab = 32 * KC * 16;            // bytes per staged table
    static_assert(2 * kTab <= G::kKBytes && 2 * kTab <= G::kVBytes, "table staging fits a ring buffer");
    __shared__ __attribute__((aligned(16))) unsigned char tst[2][2 * kTab];
    constexpr int NC = D / 16;
    constexpr int NDB = D / 32;

    const int lane = threadIdx.x % 64;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);   // 0..7
    const int grp = w >> 2, wg = w & 3;
    const int n = lane % 32, g = lane / 32;
    const int tq = p.tq;
    const float C = p.scale * kLog2e;
    const float sc = PREP ? 1.0f : C;

    // ---- tile loads: group A's waves load K, group B's V; load t of a wave fills 64
    // consecutive 16-byte slots of the tile buffer (a slot past a row's data repeats its
    // last chunk: padding, never read).
    const bool loads_k = grp == 0;
    const int nloads = loads_k ? (G::kKLoads - wg + 3) / 4 : (G::kVLoads - wg + 3) / 4;
    const int lrs = loads_k ? p.k_rs : p.v_rs;
    int voff[G::kPer];
#pragma unroll
    for (int t = 0; t < G::kPer; ++t) {
        const int sidx = (wg + 4 * t) * 64 + lane;
        const int row = loads_k ? sidx / G::kKSlots : sidx / G::kVSlots;
        const int col = sidx - row * (loads_k ? G::kKSlots : G::kVSlots);
        voff[t] = (row * lrs + 8 * min(col, G::kChunks - 1)) * 2;
    }

    // Table staging: load i of a table fills slots 64 i .. 64 i + 63 (row r = slot / KC,
    // slot s = slot % KC), and slot s of row r holds the row's chunk s ^ (r mod KC), so the
    // fragment reads below (16 lanes: 16 rows, one chunk) hit 16 distinct slots.  A slot
    // whose chunk lies past a row of half < D / 2 floats holds bytes of the next row: it is
    // never read.  (The per-lane offsets are made per item, in the prologue: kept for the
    // whole kernel they would hold registers through the tile loop.)
    unsigned char *const tslot = wg < 2 ? tst[wg] : (wg == 2 ? kb2 : vb2);

    // Per-lane LDS byte offsets of the fragment reads.
    const int k_lane = n * G::kKStride + 16 * g;
    const int j16 = lane % 16, rg = (lane % 32) / 16;
    const int v_lane = (4 * g + j16 / 4) * G::kVStride + (16 * rg + 4 * (j16 % 4)) * 2;

    // qw into LDS once; key-norm bound (the same for every item): the caller's kmax,
    // and when the call prepped k from kw, sqrt(D) max|kw| (each prepped key row is its
    // RMS-normed values times kw, turned, rounded to bf16) -- whichever is smaller.
    float kbnd = 0.f;
    if constexpr (PREP) {
        if (threadIdx.x < D) qw_s[threadIdx.x] = p.qw[threadIdx.x];
        kbnd = p.kmax;
        if (p.kwb) {
            float a = fabsf(p.kwb[lane % D]);
            if constexpr (D > 64) a = fmaxf(a, fabsf(p.kwb[64 + lane % (D - 64)]));
            const float kw_bound = __builtin_sqrtf((float)D) * max_lanes<64>(a) * (1.0f + 1.0f / 128);
            kbnd = kbnd > 0.f ? fminf(kbnd, kw_bound) : kw_bound;
        }
        // (the same in every lane; read from one so the compiler knows it is uniform and
        // keeps the branches that depend on it scalar)
        kbnd = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, kbnd)));
    }
    __syncthreads();

    // Group B runs one step behind group A inside each item's tile loop.  When the two
    // groups' slots share their query rows (mode 0) the groups run their prologues side
    // by side: B takes one barrier more after its prologue and skips the one between its
    // last matrix step and its epilogue.  Otherwise B stays one step behind across items
    // too: one barrier here, and A takes one more at the end.
    const bool together = p.mode == 0;
    if (grp == 1 && !together) __syncthreads();

    // ---- the block's items: a snake over its list.  Item r's place in the list, its
    // length class (longest first), its slot index within the pair and its pair.
    const int list = (int)blockIdx.x % p.xcds;
    const int jb = (int)blockIdx.x / p.xcds;
    struct Item {
        int idx, lcls, sub, b, kvh;
    };
    auto item_at = [&](int r) __attribute__((always_inline)) {
        Item it;
        it.idx = r * p.nbx + ((r & 1) ? p.nbx - 1 - jb : jb);
        const int per_len = p.ppx * p.nsub;
        const int lr = it.idx / per_len;
        const int rem = it.idx - lr * per_len;
        const int pl = rem / p.nsub;
        it.sub = rem - pl * p.nsub;
        it.lcls = p.nlen - 1 - lr;
        const int pair = pl * p.xcds + list;
        it.b = __builtin_amdgcn_readfirstlane(pair / p.hkv);
        it.kvh = pair - it.b * p.hkv;
        return it;
    };
    // This group's slot of an item: its q head, its query tile and the block's last one.
    auto slot_of = [&](const Item &it, int &h, int &qtile, int &qt_last) __attribute__((always_inline)) {
        if (p.mode == 0) {
            h = it.kvh * p.group + 2 * it.sub + grp;
            qtile = it.lcls;
            qt_last = it.lcls;
        } else {
            h = it.kvh * p.group + it.sub;
            qtile = 2 * it.lcls + grp;
            qt_last = 2 * it.lcls + 1;
        }
    };
    // The wave's 32 q rows of an item in the fragment layout (each load reads 32 rows);
    // rows past the query tail read as zeros.  Issued for the next item before this
    // item's output stores, so the prologue does not wait behind them.
    u32x4 raw[NC];
    auto load_q = [&](const Item &it) __attribute__((always_inline)) {
        int h, qtile, qt_last;
        slot_of(it, h, qtile, qt_last);
        const int row0w = qtile * kBM + 32 * wg;
        const int wrows = max(0, min(32, tq - row0w));
        const __amdgpu_buffer_rsrc_t qsrc =
            seq_rsrc(p.q + (int64_t)it.b * p.q_bs + (int64_t)row0w * p.q_rs + (int64_t)h * D,
                     wrows > 0 ? ((int64_t)(wrows - 1) * p.q_rs + D) * 2 : 0);
        const int qoff_lane = (n * p.q_rs + 8 * g) * 2;
#pragma unroll
        for (int c = 0; c < NC; ++c) raw[c] = __builtin_amdgcn_raw_buffer_load_b128(qsrc, qoff_lane, 32 * c, 0);
    };
    Item cur = item_at(0);
    if (cur.idx < p.items_x) load_q(cur);
    for (int r = 0;; ++r) {
        if (cur.idx >= p.items_x) break;
        const int b = cur.b;
        const int kvh = cur.kvh;
        // the sequence's keys: query i sits at key position qoff + i = tk - tq + i; with
        // per-sequence lengths tk = past[b] + tq (past[b] read as 0, and the rows NaN,
        // when it lies outside [0, pos0]).  Only tk stays live: the rest is derived.
        // (read through the scalar cache: past is read-only here and b is uniform, so the
        // read waits on no vector-memory operation -- a vector load's wait would also wait
        // for the previous item's output stores)
        const int pv = p.past ? ((const __attribute__((address_space(4))) int32_t *)p.past)[b] : 0;
        const bool bad_seq = (unsigned)pv > (unsigned)p.pos0;
        const int tk = __builtin_amdgcn_readfirstlane(p.past ? (bad_seq ? 0 : pv) + tq : p.tk);
        const int qoff = tk - tq;
        // this group's slot (q head, query tile); the block's key extent covers both slots
        int h, qtile, qt_last;
        slot_of(cur, h, qtile, qt_last);
        const int blk_last = CAUSAL ? min(tk - 1, qt_last * kBM + kBM - 1 + qoff) : tk - 1;
        const int ntiles = blk_last / kBN + 1;              // block-uniform

        const int row0w = qtile * kBM + 32 * wg;
        const int wrows = max(0, min(32, tq - row0w));
        const int rrow = row0w + n;
        const int wfirst = row0w + qoff, wlast = row0w + 31 + qoff;

        const bool paged = p.kv_pages.pages != nullptr;
        const uint16_t *src = (loads_k ? p.k : p.v) + (paged ? 0 : (int64_t)b * (loads_k ? p.k_bs : p.v_bs)) +
                              (int64_t)kvh * D;
        bool bad_page = bad_seq;          // a page id outside the pool was met (every wave
                                          // looks up the page of every tile it loads), or
                                          // the sequence's past[b] is out of range
        auto load_tile = [&](int kt, unsigned char *dst) __attribute__((always_inline)) {
            const int key0 = kt * kBN;
            __amdgpu_buffer_rsrc_t rsrc;
            if (paged) {
                const int64_t prow = pool_row(p.kv_pages, b, key0, bad_page);
                rsrc = seq_rsrc(src + prow * lrs, ((int64_t)(min(kBN, tk - key0) - 1) * lrs + D) * 2);
            } else {
                rsrc = seq_rsrc(src + (int64_t)key0 * lrs, ((int64_t)(tk - 1 - key0) * lrs + D) * 2);
            }
#pragma unroll
            for (int t = 0; t < G::kPer; ++t)
                if (t < nloads) buffer_to_lds16(rsrc, dst + (wg + 4 * t) * 1024, voff[t]);
        };

        // ======== prologue step: q, then the turn's table rows, then this group's first
        // two tiles (A: K_0, K_1; B: V_0, V_1), then q's HeadPrep.  q comes in the fragment
        // layout (each load reads 32 rows).  The tables (32 consecutive rows of each) come
        // as whole-row loads straight into LDS, staged as set out above, and are read back
        // in the fragment layout: loads that each touch 32 rows were the prologue's slowest
        // part.  The staging slots are free here: the third ring buffers are next filled
        // in softmax step 0, and the two groups' prologues either lie on either side of a
        // barrier or (mode 0) stage the same rows, so that their writes to a slot agree.
        // Constant load offsets go in the scalar offset.
        bf16x8 qf[NC];
        float shift = 0.f;
        {
            const int hc = PREP ? p.half / 16 : 0;
            if constexpr (PREP) {
                // (issued even without a turn, hc = 0: the loads then read nothing and
                // fill the slots with zeros, and the count of loads in flight stays fixed)
                const int64_t tbytes = (int64_t)wrows * p.half * 4;
                // table row of query row i: pos0 + i, or past[b] + i
                const int first = p.past ? qoff : p.pos0;
                const __amdgpu_buffer_rsrc_t crs = seq_rsrc(p.cos + (int64_t)(first + row0w) * p.half, tbytes);
                const __amdgpu_buffer_rsrc_t srs = seq_rsrc(p.sin + (int64_t)(first + row0w) * p.half, tbytes);
                // per-lane offsets, one per pattern (load i uses pattern i mod NV), and the
                // bytes per load (scalar), pinned here so they are not kept across the loop
                const int rb = pp_pin_s(RPI * p.half * 4);
                int tvoff[NV];
#pragma unroll
                for (int k = 0; k < NV; ++k) {
                    tvoff[k] = pp_pin_v((lane / KC) * (rb / RPI) + (((lane % KC) ^ ((k * RPI + lane / KC) % KC)) * 16));
                }
                // (whole offsets per lane: the range check covers the per-lane offset).  With
                // prologues side by side the two groups' waves wg stage the same rows: A
                // loads cos, B sin, and a barrier below publishes both.
                if (!together || grp == 0) {
#pragma unroll
                    for (int i = 0; i < NT; ++i)
                        pp_to_lds16(crs, tslot + 1024 * i, tvoff[i % NV] + i * rb, 0);
                }
                if (!together || grp == 1) {
#pragma unroll
                    for (int i = 0; i < NT; ++i)
                        pp_to_lds16(srs, tslot + kTab + 1024 * i, tvoff[i % NV] + i * rb, 0);
                }
            }
            load_tile(0, loads_k ? kb0 : vb0);
            if (ntiles > 1) load_tile(1, loads_k ? kb1 : vb1);
            if constexpr (PREP) {
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
                // RMS, weight and turn are linear: one multiply by the row's 1 / rms and
                // scale log2 e after the turn.
                const float f = C * __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
                // The staged tables: wait for their loads (only the tile loads issued
                // after them may still fly; with prologues side by side, a barrier then
                // publishes the other group's half), then read the lane's chunks 4c + 2g + j.
                f32x4 cv[4][2], sv[4][2];
                wait_vmcnt_upto(nloads * (ntiles > 1 ? 2 : 1));
                if (together) lds_barrier();
                const int tsw = pp_pin_v(n % KC);
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        if (2 * c < NC && c < hc) {
                            const int at = (n * KC + ((4 * c + 2 * g + j) ^ tsw)) * 16;
                            cv[c][j] = *reinterpret_cast<const f32x4 *>(tslot + at);
                            sv[c][j] = *reinterpret_cast<const f32x4 *>(tslot + kTab + at);
                        } else {
                            cv[c][j] = f32x4{1.f, 1.f, 1.f, 1.f};
                            sv[c][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                        }
                    }
                switch (hc) {
                    case 1: pp_prep_q<NC, 1>(raw, qw_s, cv, sv, g, f, qf); break;
                    case 2: pp_prep_q<NC, 2>(raw, qw_s, cv, sv, g, f, qf); break;
                    case 3: pp_prep_q<NC, 3>(raw, qw_s, cv, sv, g, f, qf); break;
                    case 4: pp_prep_q<NC, NC / 2 >= 4 ? 4 : 0>(raw, qw_s, cv, sv, g, f, qf); break;
                    default: pp_prep_q<NC, 0>(raw, qw_s, cv, sv, g, f, qf); break;
                }
                if (kbnd > 0.f) {
                    // |q| of the bf16 values the products take; Cauchy-Schwarz bounds
                    // each score by |q| kb, and the margin covers the f32 accumulation.
                    float qn = 0.f;
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const bf16x2 pr = {qf[c][2 * j], qf[c][2 * j + 1]};
                            qn = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, qn, false);
                        }
                    qn += __shfl_xor(qn, 32, 64);
                    shift = __builtin_sqrtf(qn) * kbnd * (1.0f + 1.0f / 1024);
                }
            } else {
                // q is taken as given: scaling it before the product would round it twice.
#pragma unroll
                for (int c = 0; c < NC; ++c) qf[c] = __builtin_bit_cast(bf16x8, raw[c]);
            }
        }
        // Fixed shift when every row of the wave has a score bound <= kFixedShiftMax
        // (wave-uniform); else the running maximum.
        const bool fixed = PREP && kbnd > 0.f && __builtin_amdgcn_ballot_w64(!(shift <= kFixedShiftMax)) == 0;
        float m_run = fixed ? shift : -INFINITY, l_run = 0.f;
        f32x16 s[2];
        f32x16 o[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
        if (grp == 1 && together) __syncthreads();       // B: past A's matrix step 0
        if (loads_k) __builtin_amdgcn_s_waitcnt(0);         // K_0, K_1 in LDS before A's first read
        __syncthreads();
        // Wait until at most this wave's latest batch of tile loads (nloads, or none when
        // `latest` is false) is still in flight.
        auto wait_older = [&](bool latest) __attribute__((always_inline)) {
            if (!latest || nloads == 0) {
                __builtin_amdgcn_s_waitcnt(0);
            } else if (nloads == 2) {
                ATTN_WAIT_VMCNT(2);
            } else if (nloads == 3) {
                ATTN_WAIT_VMCNT(3);
            } else if (nloads == 4) {
                ATTN_WAIT_VMCNT(4);
            } else {
                ATTN_WAIT_VMCNT(5);
            }
        };

        // A tile t is visible to this wave unless it lies wholly past its last row.
        auto visible = [&](int t) __attribute__((always_inline)) {
            return wrows > 0 && !(CAUSAL && t * kBN > wlast);
        };
        bf16x8 pf[4];
        // S^T(t) = K_t Q^T (the first product of each chain starts from zero)
        auto g1 = [&](const unsigned char *kbuf) __attribute__((always_inline)) {
            bf16x8 ka[NC][2];
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    ka[c][h2] = *reinterpret_cast<const bf16x8 *>(kbuf + k_lane + h2 * 32 * G::kKStride + 32 * c);
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    s[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c][h2], qf[c], c == 0 ? f32x16{} : s[h2], 0, 0, 0);
            // reads run four fragments ahead of the products
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * NC - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        };
        // O^T += V_t^T P(t)^T: the A fragment of (d block db, keys 16u..16u+15) is two
        // transposing reads, keys 16u + 4g + 0..3 and 16u + 8 + 4g + 0..3 (P's slot order).
        // Software-pipelined in the source: the fragments of step u+1 are read before the
        // products of step u (fences keep the scheduler from sinking the reads again).
        auto g2 = [&](const unsigned char *vbuf) __attribute__((always_inline)) {
            i16x4 vf[2][NDB][2];
            auto read_v = [&](int u, i16x4 (&f)[NDB][2]) __attribute__((always_inline)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const unsigned char *va = vbuf + v_lane + 16 * u * G::kVStride + 64 * db;
                    f[db][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(va));
                    f[db][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(va + 8 * G::kVStride));
                }
            };
            read_v(0, vf[0]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (u < 3) read_v(u + 1, vf[(u + 1) % 2]);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const i16x4 both[2] = {vf[u % 2][db][0], vf[u % 2][db][1]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pf[u], o[db], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // P(t) = exp2((S(t) - m) sc): mask, running maximum, weights as the B operand (step
        // u covers keys 16u..16u+15, registers 8(u%2).. of block u/2), row sum.
        auto sm = [&](int t) __attribute__((always_inline)) {
            const int key0 = t * kBN;
            const bool need_mask = (key0 + kBN > tk) || (CAUSAL && key0 + kBN - 1 > wfirst);
            if (need_mask) {
                // Keys past this lane's row (its causal diagonal) or past the sequence get
                // -inf.  Register 4i+jj of block h2 holds key key0 + 32 h2 + 8 i + 4 g + jj;
                // the masked offsets form a 64-bit mask, read back with one bit-field
                // extract (0 or -1) and applied with one bit-field insert per register --
                // no compares, which would each hold a scalar mask register.
                const int lim = (CAUSAL ? min(tk - 1, rrow + qoff) : tk - 1) - (key0 + 4 * g);
                const int nvis = min(max(lim + 1, 0), 64);
                const uint64_t masked = nvis >= 64 ? 0ull : (~0ull << nvis);
                const uint32_t mw[2] = {(uint32_t)masked, (uint32_t)(masked >> 32)};
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)mw[h2], 8 * (i / 4) + (i % 4), 1);
                        s[h2][i] = __uint_as_float((m & 0xFF800000u) | (~m & __float_as_uint(s[h2][i])));
                    }
            }
            if (!fixed) {
                float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
                for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[0][i], s[0][i + 1]));
#pragma unroll
                for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[1][i], s[1][i + 1]));
                mx = fmaxf(mx, pp_lane_pair(mx, g));             // tile maximum of the row
                const bool first = m_run == -INFINITY;
                const bool raise = first ? mx > -INFINITY : (mx - m_run) * sc > kRaiseAbove;
                if (__builtin_amdgcn_ballot_w64(raise)) {        // wave-uniform, rare
                    const float alpha = first || !raise ? 1.f : fast_exp2((m_run - mx) * sc);
                    l_run *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
                    if (raise) m_run = mx;
                }
            }
            // Weights.  With the fixed bound every score of the row lies in [-b, b], b <=
            // kFixedShiftMax (base 2), so 2^s is a normal f32 and bf16 number: no shift is
            // needed (any common factor cancels between the weighted sum and the row sum),
            // one exponential a weight.  Otherwise exp2(s sc - m sc), one fused multiply-add
            // more (the shift is 0 until the first visible key, when every weight is 0).
            // (two copies of the loop, so the choice is one branch, not a select per weight)
            const float msc = m_run == -INFINITY ? 0.f : m_run * sc;
            auto weights = [&](auto bare) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float e8[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float x = s[u / 2][8 * (u % 2) + i];
                    e8[i] = fast_exp2(decltype(bare)::value ? x : __builtin_fmaf(x, sc, -msc));
                }
                uint4 pk;
                pk.x = pack_bf16x2(e8[0], e8[1]);
                pk.y = pack_bf16x2(e8[2], e8[3]);
                pk.z = pack_bf16x2(e8[4], e8[5]);
                pk.w = pack_bf16x2(e8[6], e8[7]);
                // Row sum of the f32 weights by plain adds: v_dot2_f32_bf16 runs on the
                // matrix cores' datapath and would wait for the other group's products.
                // (The P V product takes the bf16 roundings, which differ from these by at
                // most 2^-9 relative each.)
                l_run += ((e8[0] + e8[1]) + (e8[2] + e8[3])) + ((e8[4] + e8[5]) + (e8[6] + e8[7]));
                pf[u] = __builtin_bit_cast(bf16x8, pk);
            }
            };
            if (fixed)
                weights(std::true_type());
            else
                weights(std::false_type());
        };

        // ======== tile steps.  Every wave runs, per tile period t = 0 .. ntiles, a
        // matrix step (P(t-1) V_{t-1}, then S(t): the weights free their registers
        // before the K fragments take theirs), a barrier, a softmax step (P(t); the
        // epilogue at t = ntiles), a barrier.  Group B runs one step behind A, so B's
        // matrix step runs beside A's softmax step and the other way round (phases
        // between barriers; mode 0, prologues side by side):
        //   A: prologue | M0 | S0 | ... | MT   | epilogue     | prologue | M0 | S0 ...
        //   B: prologue |    | M0 | ... | ST-1 | MT, epilogue | prologue |    | M0 ...
        // (other modes, prologues one after the other:
        //   A: prologue | M0       | S0 | ... | MT   | epilogue | prologue | M0       ...
        //   B:          | prologue | M0 | ... | ST-1 | MT       | epilogue | prologue ...)
        // Tiles live in rings of three LDS buffers (tile t in buffer t mod 3).  A issues
        // K_{t+2} as its softmax step t starts (the buffer held K_{t-1}, whose last
        // reader, B's matrix step t-1, ended two barriers before) and, at the end of that
        // step, waits for K_{t+1} (issued a period earlier), which A's matrix step t+1
        // reads next.  B issues V_{t+2} as its softmax step t starts (the buffer
        // held V_{t-1}, last read by B's matrix step t, a barrier before) and, at the end
        // of its matrix step t+1, waits for V_{t+1}, which A's matrix step t+2 reads
        // next.  So each tile has about a period and a half to arrive.
        auto mstep = [&](int t, const unsigned char *kcur, const unsigned char *vprev) __attribute__((always_inline)) {
            __builtin_amdgcn_s_setprio(1);
            if (t >= 1 && visible(t - 1)) g2(vprev);
            if (t < ntiles && visible(t)) g1(kcur);
            __builtin_amdgcn_s_setprio(0);
            if (!loads_k) wait_older(t + 1 < ntiles);      // V_t in LDS (V_{t+1} may fly)
        };
        auto sstep = [&](int t, unsigned char *knext2, unsigned char *vnext2) __attribute__((always_inline)) {
            // Both groups issue their loads as their softmax step starts, so each block
            // phase carries one group's load issue and no matrix step carries any.
            if (t + 2 < ntiles) load_tile(t + 2, loads_k ? knext2 : vnext2);
            if (t < ntiles && visible(t)) sm(t);
            if (loads_k) wait_older(t + 2 < ntiles);       // K_{t+1} in LDS (K_{t+2} may fly)
        };
        // (periods 0 .. ntiles - 1 here; the matrix step of period ntiles ends the loop)
        for (int t = 0;; t += 3) {
            mstep(t, kb0, vb2);
            if (t == ntiles) break;
            __syncthreads();
            sstep(t, kb2, vb2);
            __syncthreads();
            mstep(t + 1, kb1, vb0);
            if (t + 1 == ntiles) break;
            __syncthreads();
            sstep(t + 1, kb0, vb0);
            __syncthreads();
            mstep(t + 2, kb2, vb1);
            if (t + 2 == ntiles) break;
            __syncthreads();
            sstep(t + 2, kb1, vb1);
            __syncthreads();
        }
        // The softmax step of period ntiles holds no tile work: A waits for its last
        // loads, and the epilogue follows (for B in mode 0 without a barrier).
        if (!(grp == 1 && together)) __syncthreads();
        if (loads_k) __builtin_amdgcn_s_waitcnt(0);
        const Item nxt = item_at(r + 1);
        if (nxt.idx < p.items_x) load_q(nxt);

        // ---- epilogue (in the softmax step of period ntiles, or for B in mode 0 right
        // after its last matrix step): divide by the row sum, round once to bf16, store.
        // The wave's 32 x D output tile goes through LDS (chunk c of row r at slot
        // c ^ (r mod KC), as the tables), so that each store writes whole rows (a store of
        // the fragment layout touches 32 rows).  Staging: A in tst (no table is staged
        // until the next prologue), B in the K ring (mode 0: no matrix step reads K from
        // the last one on) or the V ring (other modes: the epilogue lies between B's last
        // matrix step and its next prologue); two waves a buffer.  Rows past the query
        // tail fall outside the store's range and are dropped.
        {
            const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
            const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
            // A bad page: quiet-NaN bf16 bits (set as integers: this file is built without
            // NaN semantics).
            const uint32_t nan_mask = bad_page ? 0xFFFFFFFFu : 0u;
            unsigned char *const est = (grp == 0 ? tst[wg >> 1] : together ? ((wg >> 1) ? kb1 : kb0) : ((wg >> 1) ? vb1 : vb0)) +
                                       (wg & 1) * kTab;
            const int esw = pp_pin_v(n % KC);          // (made here, not kept across the loop)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint2 u;
                    u.x = pack_bf16x2(o[db][4 * i] * inv, o[db][4 * i + 1] * inv);
                    u.y = pack_bf16x2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
                    u.x = (u.x & ~nan_mask) | (0x7FC07FC0u & nan_mask);
                    u.y = (u.y & ~nan_mask) | (0x7FC07FC0u & nan_mask);
                    // columns 32 db + 8 i + 4 g .. + 3 of row n: chunk 4 db + i, half g
                    *reinterpret_cast<uint2 *>(est + n * (2 * D) + (((4 * db + i) ^ esw) * 16) + 8 * g) = u;
                }
            const __amdgpu_buffer_rsrc_t ors =
                seq_rsrc(p.out + (int64_t)b * p.o_bs + (int64_t)row0w * p.o_rs + (int64_t)h * D,
                         wrows > 0 ? ((int64_t)(wrows - 1) * p.o_rs + D) * 2 : 0);
            // (the whole offset per lane, scalar offset 0: the range check then sees it, and
            // the compiler keeps the wait a store of more than 8 bytes needs before its data
            // registers are written again -- it drops that wait for a register scalar offset)
            const int rl = pp_pin_v(lane / KC), cl = pp_pin_v(lane % KC);
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                const int r = k * RPI + rl;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(est + r * (2 * D) + ((cl ^ (r % KC)) * 16));
                __builtin_amdgcn_raw_buffer_store_b128(v, ors, (r * p.o_rs + 8 * cl) * 2, 0, 0);
            }
        }
        __syncthreads();
        cur = nxt;
    }
    if (grp == 0 && !together) __syncthreads();
}

int cu_count() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

template <int D, bool CAUSAL>
hipError_t launch_bf16_d(const PrefillLaunch &a, hipStream_t stream) {
    const int64_t nq_tiles = (a.seq + kBM - 1) / kBM;
    const int64_t group = a.hq / a.hkv, pairs = a.batch * a.hkv;
    PPArgs p{};
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.out = static_cast<uint16_t *>(a.out);
    p.qw = a.qw; p.cos = a.cos; p.sin = a.sin; p.kwb = a.kwb;
    p.q_bs = a.q_bs; p.k_bs = a.k_bs; p.v_bs = a.v_bs; p.o_bs = a.o_bs;
    p.q_rs = (int)a.q_rs; p.k_rs = (int)a.k_rs; p.v_rs = (int)a.v_rs; p.o_rs = (int)a.o_rs;
    p.kv_pages = a.kv_pages;
    p.past = a.past;
    p.tq = (int)a.seq; p.tk = (int)a.tk; p.half = (int)a.half; p.pos0 = (int)a.pos0;
    p.eps = a.eps; p.scale = a.scale; p.kmax = a.kmax;
    p.mode = group % 2 == 0 ? 0 : 1;
    p.group = (int)group;
    p.hkv = (int)a.hkv;
    p.nsub = (int)(p.mode == 0 ? group / 2 : group);
    p.nlen = (int)(p.mode == 0 ? nq_tiles : (nq_tiles + 1) / 2);
    const int cus = cu_count();
    if (pairs % kXcds == 0 && cus % kXcds == 0) {
        p.xcds = kXcds;
        p.ppx = (int)(pairs / kXcds);
    } else {
        p.xcds = 1;
        p.ppx = (int)pairs;
    }
    const int64_t items_x = (int64_t)p.nlen * p.ppx * p.nsub;
    if (items_x >= ((int64_t)1 << 31) || a.tk >= ((int64_t)1 << 31) - kBM || a.pos0 + a.seq >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    p.items_x = (int)items_x;
    p.nbx = (int)std::min<int64_t>(cus / p.xcds, items_x);
    const dim3 grid((unsigned)(p.nbx * p.xcds));
    if (a.prep_q)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, true>), grid, dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, false>), grid, dim3(512), 0, stream, p);
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
