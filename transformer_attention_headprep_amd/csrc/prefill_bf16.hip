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
//   O^T += V^T P^T (A = V^T tile from LDS, B = P straight from the S^T registers)
// With that layout the row maximum is a max over a lane's own 32 scores plus one
// exchange with lane ^ 32, and the rescale of O needs no exchange at all.
//
// Pipeline: two LDS tile buffers; while a tile is consumed, the next one is already
// in flight from HBM into registers, and is written to the other buffer afterwards,
// so there is one barrier per tile.  Two blocks fit a CU (2 waves per SIMD), so the
// softmax arithmetic of one wave overlaps the matrix products of the other.
//
// Online softmax in base-2 units.  A prepped q (computed in f32 anyway) is multiplied
// by scale log2 e before it is rounded to bf16, and every S^T accumulation starts from
// -m (the row's running maximum, held in 16 registers), so the matrix core returns
// s log2 e - m directly and the weights are a bare v_exp_f32 of the accumulator.  A q
// given without HeadPrep is used as it is (rescaling it would round it a second time)
// and the exponent takes one multiply by scale log2 e instead.  The running maximum is only
// raised when a tile's maximum exceeds it by more than 8 (base 2): the weights
// 2^(s - m) then stay below 256, which f32 sums and bf16 weights hold exactly as well
// as weights below 1, and the rescale of O (64 multiplies a lane) is skipped on almost
// every tile.  The result is the same softmax: numerator and denominator use the same
// m.  The row sum adds the bf16-rounded weights that the P V product uses
// (v_dot2_f32_bf16), so numerator and denominator match.
//
// K and V tiles are read with buffer loads whose descriptor starts at the tile and
// ends at the sequence: rows past the end read as zero with no branch, and the tile
// offset is scalar arithmetic.
//
// The q prologue applies HeadPrep (RMS, qw, split-half turn at the row's position)
// in registers before rounding q to bf16; it needs half to be 0 or a multiple of 16
// (then every turned pair sits in one lane).  Other halves are prepped by the prep
// kernel beforehand.
//
// LDS: K is stored row-major [key][d] with rows padded by 16 bytes (conflict-free
// 16-byte reads down a column).  V is stored transposed [d][key] so that a lane's
// 8 keys for one d are 16 contiguous bytes; the 16-byte chunks of a row are XOR-
// swizzled by the row so that both the transposing writes and the reads spread over
// the banks.  Keys inside each 16-key group are placed in the order the S^T
// accumulator registers hold them (bits 2 and 3 of the key index swapped), so P needs
// no shuffling before the second product.
//
// Block order: longest causal query tiles first; when the (batch, kv head) pairs
// divide evenly over the 8 XCDs, every pair's blocks go to one XCD (blocks are
// dealt to XCDs round-robin), so its K/V stay in that XCD's L2.
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

__device__ __forceinline__ int vt_swizzle(int row) { return (row ^ (row >> 3)) & 7; }

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

template <int D>
struct TileBuf {
    static constexpr int kStride = D + 8;                 // bf16 elements per K row
    uint16_t k[kBN * kStride];
    uint16_t vt[D * kBN];                                // [d][64 keys], 128-byte rows
};

// One tile's K and V as this thread moves them: KL 16-byte pieces of K, and 4 keys x
// 8 values of V (V is transposed on its way into LDS).
template <int D>
struct Staged {
    static constexpr int KL = kBN * D / 8 / 256;
    uint4 k[KL];
    uint4 v[4];
};

// Buffer descriptor over `bytes` bytes from `base` (raw, untyped; reads past the end
// return zero).
// The arguments are block-uniform; readfirstlane puts the descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *base, int64_t bytes) {
    const int n = bytes > 0 ? (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF) : 0;
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *sbase = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(sbase, (short)0, __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// Loads the 64-key tile that starts at key0; the descriptors end with the sequence's
// last row, so keys past the sequence read as zero.
template <int D>
__device__ __forceinline__ void load_tile(Staged<D> &st, const uint16_t *kbase, const uint16_t *vbase,
                                          int k_rs, int v_rs, int key0, int seq, int tid) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase + (int64_t)key0 * k_rs, ((int64_t)(seq - 1 - key0) * k_rs + D) * 2);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vbase + (int64_t)key0 * v_rs, ((int64_t)(seq - 1 - key0) * v_rs + D) * 2);
#pragma unroll
    for (int it = 0; it < Staged<D>::KL; ++it) {
        const int idx = it * 256 + tid;
        const int key = idx / (D / 8), seg = idx % (D / 8);
        st.k[it] = buffer_load16(rk, (key * k_rs + 8 * seg) * 2);
    }
    if (tid < (kBN / 4) * (D / 8)) {
        const int seg = tid % (D / 8), quad = tid / (D / 8);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) st.v[jj] = buffer_load16(rv, ((4 * quad + jj) * v_rs + 8 * seg) * 2);
    }
}

template <int D>
__device__ __forceinline__ void store_tile(TileBuf<D> &buf, const Staged<D> &st, int tid) {
    constexpr int KS = TileBuf<D>::kStride;
#pragma unroll
    for (int it = 0; it < Staged<D>::KL; ++it) {
        const int idx = it * 256 + tid;
        const int key = idx / (D / 8), seg = idx % (D / 8);
        *reinterpret_cast<uint4 *>(&buf.k[key * KS + 8 * seg]) = st.k[it];
    }
    if (tid < (kBN / 4) * (D / 8)) {
        const int seg = tid % (D / 8), quad = tid / (D / 8);
        const int pq = (quad & ~3) | ((quad & 1) << 1) | ((quad >> 1) & 1);
        const uint32_t wd[4][4] = {{st.v[0].x, st.v[0].y, st.v[0].z, st.v[0].w},
                                   {st.v[1].x, st.v[1].y, st.v[1].z, st.v[1].w},
                                   {st.v[2].x, st.v[2].y, st.v[2].z, st.v[2].w},
                                   {st.v[3].x, st.v[3].y, st.v[3].z, st.v[3].w}};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                const int row = 8 * seg + 2 * e + hi;
                // pack value (row) of keys 4quad .. 4quad+3: low halves (even d) or high halves (odd d)
                const uint32_t sel = hi == 0 ? 0x05040100u : 0x07060302u;
                const uint32_t lo01 = __builtin_amdgcn_perm(wd[1][e], wd[0][e], sel);
                const uint32_t lo23 = __builtin_amdgcn_perm(wd[3][e], wd[2][e], sel);
                const int chunk = (pq >> 1) ^ vt_swizzle(row);
                *reinterpret_cast<uint2 *>(&buf.vt[row * kBN + chunk * 8 + (pq & 1) * 4]) = make_uint2(lo01, lo23);
            }
        }
    }
}

template <int D, bool CAUSAL, bool PREP>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(const PrefillLaunch p) {
    __shared__ TileBuf<D> bufs[2];
    constexpr int KS = TileBuf<D>::kStride;
    constexpr int NC = D / 16;       // 16-wide d chunks of the q.k product
    constexpr int NDB = D / 32;      // 32-wide d blocks of the output

    const int tid = threadIdx.x;
    const int w = tid / 64, lane = tid % 64;
    const int n = lane % 32, g = lane / 32;

    // ---- which (batch, q head, query tile) this block owns
    const int nq_tiles = (int)((p.seq + kBM - 1) / kBM);
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
    const bool row_ok = r < p.seq;

    const int64_t last_key = CAUSAL ? min<int64_t>(p.seq - 1, (int64_t)qtile * kBM + kBM - 1) : p.seq - 1;
    const int ntiles = (int)(last_key / kBN) + 1;
    const uint16_t *kbase = static_cast<const uint16_t *>(p.k) + (int64_t)b * p.seq * p.k_rs + (int64_t)kvh * D;
    const uint16_t *vbase = static_cast<const uint16_t *>(p.v) + (int64_t)b * p.seq * p.v_rs + (int64_t)kvh * D;

    // First tile on its way before the q prologue.
    const int seq = (int)p.seq, k_rs = (int)p.k_rs, v_rs = (int)p.v_rs;
    Staged<D> st;
    load_tile<D>(st, kbase, vbase, k_rs, v_rs, 0, seq, tid);

    const float C = p.scale * kLog2e;       // q is scaled by this before it is rounded

    // ---- q prologue: load this lane's 64 (or 32) values of its row, HeadPrep, bf16.
    bf16x8 qf[NC];
    {
        const uint16_t *qrow = static_cast<const uint16_t *>(p.q) +
                               ((int64_t)b * p.seq + (row_ok ? r : 0)) * p.q_rs + (int64_t)h * D;
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

    store_tile<D>(bufs[0], st, tid);
    __syncthreads();

    for (int kt = 0; kt < ntiles; ++kt) {
        const int key0 = kt * kBN;
        const TileBuf<D> &buf = bufs[kt & 1];
        const bool more = kt + 1 < ntiles;
        if (more) load_tile<D>(st, kbase, vbase, k_rs, v_rs, key0 + kBN, seq, tid);

        // S^T = K Q^T - m for 2 blocks of 32 keys (two independent accumulation chains).
        f32x16 s[2];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&buf.k[(kb * 32 + n) * KS + 16 * c + 8 * g]);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], c == 0 ? bias : s[kb], 0, 0, 0);
            }
        }
        // Mask: register 4i+jj of block kb holds key key0 + 32 kb + 8 i + 4 g + jj.
        const int row = (int)r;
        const bool need_mask = (key0 + kBN > seq) || (CAUSAL && key0 + kBN - 1 > qtile * kBM);
        if (need_mask) {
            const int lim = CAUSAL ? min(seq - 1, row) : seq - 1;   // last visible key
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = key0 + 32 * kb + 8 * (i / 4) + 4 * g + (i % 4);
                    if (j > lim) s[kb][i] = -INFINITY;
                }
        }
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[0][i], s[0][i + 1]));
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[1][i], s[1][i + 1]));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));               // tile max of s - m
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

        // P as the B operand: step u covers keys 16u..16u+15 (registers 8(u%2).. of block u/2).
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
        // O^T += V^T P^T (the NDB output blocks are independent chains)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int vrow = 32 * db + n;
                const int chunk = (2 * u + g) ^ vt_swizzle(vrow);
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&buf.vt[vrow * kBN + chunk * 8]);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[u], o[db], 0, 0, 0);
            }
        }
        if (more) store_tile<D>(bufs[(kt + 1) & 1], st, tid);
        __syncthreads();
    }

    // ---- epilogue: divide by the row sum, round once to bf16, store.
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (row_ok) {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        uint16_t *orow = static_cast<uint16_t *>(p.out) + ((int64_t)b * p.seq + r) * p.o_rs + (int64_t)h * D;
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
    if (a.prep_q)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, false>), grid, dim3(256), 0, stream, a);
}

}  // namespace

bool prefill_fuses_half(int64_t d, int64_t half, bool bf16) {
    if (!bf16) return half == 0 || 2 * half == d;
    return half == 0 || half % 16 == 0;   // pairs 1, 2, 3 or 4 chunks of 16 apart
}

hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t stream) {
    if (!a.bf16) return launch_prefill_f32(a, stream);
    if (a.d == 64) {
        if (a.causal) launch_bf16_d<64, true>(a, stream); else launch_bf16_d<64, false>(a, stream);
    } else {
        if (a.causal) launch_bf16_d<128, true>(a, stream); else launch_bf16_d<128, false>(a, stream);
    }
    return hipGetLastError();
}

}  // namespace attn
