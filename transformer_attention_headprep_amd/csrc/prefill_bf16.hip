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
// one barrier per tile.  The buffer descriptor of a tile ends with the sequence, so
// keys past its end arrive as zeros.  K rows are stored 16 bytes wider than their data
// and V rows 64 bytes wider (the extra slots are filled by the same loads): K row
// pitches step 4 banks, so the 16-byte reads of 16 consecutive key rows cover all 64
// banks once; V row pitches step 16 banks, so the transposing reads of 4 key rows x 64
// bytes by 32 lanes do too.  Every LDS offset is then an immediate.  Two blocks fit a
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

extern __shared__ __attribute__((aligned(16))) unsigned char prefill_smem[];

// The value held by lane ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float lane_pair(float x, int g) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(g == 0 ? r[1] : r[0]);
}

// Split-half turn of a lane's q values held as NC chunks of 8 (chunk c = d 16c + 8g ..):
// chunk c < HC pairs with chunk c + HC (half = 16 HC), using table entries d0 .. d0 + 7.
template <int NC, int HC>
__device__ __forceinline__ void turn_chunks(float (&x)[NC][8], const float *cr, const float *sr, int g) {
    if constexpr (HC >= 1 && 2 * HC <= NC) {
#pragma unroll
        for (int c = 0; c < HC; ++c) {
            const int d0 = 16 * c + 8 * g;
            const float4 c0 = *reinterpret_cast<const float4 *>(cr + d0);
            const float4 c1 = *reinterpret_cast<const float4 *>(cr + d0 + 4);
            const float4 s0 = *reinterpret_cast<const float4 *>(sr + d0);
            const float4 s1 = *reinterpret_cast<const float4 *>(sr + d0 + 4);
            const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = x[c][e], b = x[c + HC][e];
                x[c][e] = a * cv[e] - b * sv[e];
                x[c + HC][e] = b * cv[e] + a * sv[e];
            }
        }
    }
}

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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_bf16_kernel(const PrefillLaunch p) {
    typedef Geo<D> G;
    unsigned char *smem = prefill_smem;                                  // 2 tile buffers
    constexpr int NC = D / 16;       // 16-wide d chunks of the q.k product
    constexpr int NDB = D / 32;      // 32-wide d blocks of the output

    const int tid = threadIdx.x;
    const int w = tid / 64, lane = tid % 64;
    const int n = lane % 32, g = lane / 32;

    // ---- which (batch, q head, query tile) this block owns
    const int nq_tiles = (int)((p.seq + kBM - 1) / kBM);
    const int tq = (int)p.seq, tk = (int)p.tk, qoff = tk - tq;   // query i sits at key position i + qoff
    const int group = (int)(p.hq / p.hkv);
    const int pairs = (int)(p.batch * p.hkv);
    int b, h, qtile;
    {
        const int i = blockIdx.x;
        int pair, hg;
        if (pairs % kXcds == 0) {
            const int ppx = pairs / kXcds;                 // pairs per XCD
            const int x = i % kXcds;
            const int j = i / kXcds;
            const int per_tile = ppx * group;
            qtile = nq_tiles - 1 - j / per_tile;
            const int rem = j % per_tile;
            pair = x + kXcds * (rem / group);
            hg = rem % group;
        } else {
            const int per_tile = pairs * group;
            qtile = nq_tiles - 1 - i / per_tile;
            const int rem = i % per_tile;
            pair = rem / group;
            hg = rem % group;
        }
        b = pair / (int)p.hkv;
        h = (pair % (int)p.hkv) * group + hg;
    }
    const int kvh = h / group;

    const int64_t r = (int64_t)qtile * kBM + 32 * w + n;
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
    const uint16_t *src = static_cast<const uint16_t *>(loads_k ? p.k : p.v) +
                          (int64_t)b * (loads_k ? p.k_bs : p.v_bs) + (int64_t)kvh * D;
    const int slots = loads_k ? G::kKSlots : G::kVSlots;
    int voff[G::kPerWave];
#pragma unroll
    for (int t = 0; t < G::kPerWave; ++t) {
        const int sidx = (wl + 2 * t) * 64 + lane;
        const int row = sidx / slots, col = sidx % slots;
        voff[t] = (int)(row * rs + 8 * min(col, G::kChunks - 1)) * 2;
    }
    auto load_tile = [&](int kt, int bsel) {
        const int key0 = kt * kBN;
        const __amdgpu_buffer_rsrc_t rsrc = seq_rsrc(src + (int64_t)key0 * rs, ((int64_t)(tk - 1 - key0) * rs + D) * 2);
        unsigned char *dst = smem + bsel * G::kBufBytes + (loads_k ? 0 : G::kKBytes);
#pragma unroll
        for (int t = 0; t < G::kPerWave; ++t) {
            if (t < nloads)
                buffer_to_lds16(rsrc, dst + (wl + 2 * t) * 1024, voff[t]);
        }
    };

    // First tile on its way before the q prologue.
    load_tile(0, 0);

    const float C = p.scale * kLog2e;       // q is scaled by this before it is rounded

    // ---- q prologue: load this lane's 64 (or 32) values of its row, HeadPrep, bf16.
    bf16x8 qf[NC];
    {
        const uint16_t *qrow = static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_bs +
                               (row_ok ? r : 0) * p.q_rs + (int64_t)h * D;
        uint4 raw[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
            raw[c] = row_ok ? *reinterpret_cast<const uint4 *>(qrow + 16 * c + 8 * g) : make_uint4(0, 0, 0, 0);
        if constexpr (PREP) {
            float x[NC][8];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                unpack_bf16x2(raw[c].x, x[c][0], x[c][1]);
                unpack_bf16x2(raw[c].y, x[c][2], x[c][3]);
                unpack_bf16x2(raw[c].z, x[c][4], x[c][5]);
                unpack_bf16x2(raw[c].w, x[c][6], x[c][7]);
            }
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += x[c][e] * x[c][e];
            ss += __shfl_xor(ss, 32, 64);
            const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / D) + p.eps);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float4 w0 = *reinterpret_cast<const float4 *>(p.qw + 16 * c + 8 * g);
                const float4 w1 = *reinterpret_cast<const float4 *>(p.qw + 16 * c + 8 * g + 4);
                const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) x[c][e] = x[c][e] * inv * wv[e];
            }

            const int hc = (int)p.half / 16;     // turned pairs are hc chunks apart
            if (hc > 0 && row_ok) {
                const float *cr = p.cos + (p.pos0 + r) * p.half;
                const float *sr = p.sin + (p.pos0 + r) * p.half;
                // hc is a run-time value; dispatch to unrolled code so x stays in registers.
                switch (hc) {
                    case 1: turn_chunks<NC, 1>(x, cr, sr, g); break;
                    case 2: turn_chunks<NC, 2>(x, cr, sr, g); break;
                    case 3: turn_chunks<NC, 3>(x, cr, sr, g); break;
                    default: turn_chunks<NC, NC / 2>(x, cr, sr, g); break;
                }
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                uint4 u;
                u.x = pack_bf16x2(x[c][0] * C, x[c][1] * C);
                u.y = pack_bf16x2(x[c][2] * C, x[c][3] * C);
                u.z = pack_bf16x2(x[c][4] * C, x[c][5] * C);
                u.w = pack_bf16x2(x[c][6] * C, x[c][7] * C);
                qf[c] = __builtin_bit_cast(bf16x8, u);
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
    float m_run = -INFINITY, l_run = 0.f;   // l_run: this lane's share of the row sum
    f32x16 bias;                             // -m_run (0 until the first visible key)
#pragma unroll
    for (int i = 0; i < 16; ++i) bias[i] = 0.f;
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

    for (int kt = 0; kt < ntiles; ++kt) {
        const int key0 = kt * kBN;
        const int bsel = kt & 1;
        if (kt + 1 < ntiles) load_tile(kt + 1, bsel ^ 1);
        const unsigned char *buf = smem + bsel * G::kBufBytes;

        // S^T = K Q^T - m for 2 blocks of 32 keys (two independent accumulation chains).
        f32x16 s[2];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(buf + k_lane + kb * 32 * G::kKStride + 32 * c);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], c == 0 ? bias : s[kb], 0, 0, 0);
            }
        }
        // Mask: register 4i+jj of block kb holds key key0 + 32 kb + 8 i + 4 g + jj.
        const bool need_mask = (key0 + kBN > tk) || (CAUSAL && key0 + kBN - 1 > qtile * kBM + qoff);
        if (need_mask) {
            const int lim = (CAUSAL ? min(tk - 1, (int)r + qoff) : tk - 1) - (key0 + 4 * g);   // last visible
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kb + 8 * (i / 4) + (i % 4) > lim) s[kb][i] = -INFINITY;
        }
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[0][i], s[0][i + 1]));
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[1][i], s[1][i + 1]));
        mx = fmaxf(mx, lane_pair(mx, g));                     // tile max of s - m
        const bool first = m_run == -INFINITY;
        const bool raise = first ? mx > -INFINITY : mx * sc > kRaiseAbove;
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
    }

    // ---- epilogue: divide by the row sum, round once to bf16, store.
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (row_ok) {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        uint16_t *orow = static_cast<uint16_t *>(p.out) + (int64_t)b * p.o_bs + r * p.o_rs + (int64_t)h * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint2 u;
                u.x = pack_bf16x2(o[db][4 * i] * inv, o[db][4 * i + 1] * inv);
                u.y = pack_bf16x2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * i + 4 * g) = u;
            }
    }
}

template <int D, bool CAUSAL>
void launch_bf16_d(const PrefillLaunch &a, hipStream_t stream) {
    const int64_t nq_tiles = (a.seq + kBM - 1) / kBM;
    const dim3 grid((unsigned)(nq_tiles * a.batch * a.hq));
    const size_t lds = 2 * Geo<D>::kBufBytes;
    if (a.prep_q)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, true>), grid, dim3(256), lds, stream, a);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, false>), grid, dim3(256), lds, stream, a);
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
    if (a.d == 64) {
        if (a.causal) launch_bf16_d<64, true>(a, stream); else launch_bf16_d<64, false>(a, stream);
    } else {
        if (a.causal) launch_bf16_d<128, true>(a, stream); else launch_bf16_d<128, false>(a, stream);
    }
    return hipGetLastError();
}

}  // namespace attn
