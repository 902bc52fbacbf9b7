// rows8.hip -- attentionRows' quantised path: Q K^T on INT8 and P V on E4M3 (gizml:netops
// reference page, Functions > attentionRows with `quantized`: SageAttention's split of the
// two products), with the head norm and rotary in the quantizing pass.
//
// Quantizing pass (rows8_quant_kernel, rows8_vt_kernel), per (64-row tile of a group, head):
//   q: HeadPrep in f32, then int8 per (row, head): s = amax / 127, c = rint(x (1/s)).
//   k: HeadPrep in f32, then int8 per (tile, head): one scale for the tile's 64 keys.
//   v: E4M3 per (group, head): s = amax / 448 over the group (the first kernel leaves each
//      tile's amax, the second takes their largest), values rounded to nearest (ties even) by
//      v_cvt_pk_fp8_f32, stored transposed ([d][64 keys]) with the keys of a tile in the
//      order the P V product consumes them.
// Every decision runs in f32 in the order written (correctly rounded division, no
// contraction: the file is compiled with -ffp-contract=off).
//
// Attention (attn8_kernel): a block owns 128 query rows of one (group, head); 4 waves of 32
// rows; key tiles of 64 go HBM -> LDS by buffer loads that write LDS directly, double
// buffered, as in the bf16 prefill.  Both products are transposed so a lane holds one
// query row:
//   S^T = K Q^T on v_mfma_i32_32x32x32_i8 (lane (row r, half g) of an operand holds its
//       row's bytes 16g .. 16g + 15 of a 32-wide k step), then scaled in f32 by the query
//       row's scale, the tile's key scale, and scale log2 e;
//   an online softmax whose running max moves with every larger score, so the weights
//       2^(s - m) 448 fill the E4M3 range (largest 448, smallest normal 2^-6 448^-1 of it);
//       the row sum adds the weights before they are rounded;
//   O^T += V^T P^T on v_mfma_f32_32x32x64_f8f6f4 (E4M3 both), the lane's 32 weights being
//       its B fragment in register order, which is why the stored V^T puts key
//       32 (b / 16) + 8 ((b % 16) / 4) + 4 g + b % 4 at position 32 g + b of a tile.
// The output is O / l times the group's value scale, rounded once to bf16.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;          // keys per tile (and per int8 key scale)
constexpr int kBM = 128;           // query rows per attention block

__device__ __forceinline__ float lane_pair8(float x, int g) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(g == 0 ? r[1] : r[0]);
}

// ------------------------------------------------------------------ quantizing pass

// HeadPrep of one row held as lo[4] (values 4 li ..) and hi[4] (values D/2 + 4 li ..) by the
// LPR lanes of the row.  MODE 0: none; 1: split halves (half = D/2, or 0: norm and weight
// only); 2: adjacent pairs.  tc / ts: the row's table entries this lane needs, loaded
// beforehand -- MODE 1: entries 4 li .. 4 li + 3; MODE 2: entries 2 li, 2 li + 1 (pairs
// of lo) and D/4 + 2 li, D/4 + 2 li + 1 (pairs of hi), used only below `half`.
template <int D, int MODE>
__device__ __forceinline__ void prep_row(float (&lo)[4], float (&hi)[4], int li, const float *w, const f32x4 &tc,
                                         const f32x4 &ts, int half, float eps) {
    constexpr int LPR = D / 8;
    if constexpr (MODE == 0) return;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) ss += lo[i] * lo[i] + hi[i] * hi[i];
    ss = sum_lanes<LPR>(ss);
    const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / D) + eps);
    const int el = 4 * li, eh = D / 2 + 4 * li;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = lo[i] * inv * w[el + i];
        hi[i] = hi[i] * inv * w[eh + i];
    }
    if (half == 0) return;
    if constexpr (MODE == 1) {          // half = D / 2: value e with e + D / 2, entry e
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float c = tc[i], s = ts[i], a = lo[i], b = hi[i];
            lo[i] = a * c - b * s;
            hi[i] = b * c + a * s;
        }
    } else {                            // pairs (2j, 2j + 1), entry j < half
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            const int jl = (el + i) / 2, jh = (eh + i) / 2;
            if (jl < half) {
                const float c = tc[i / 2], s = ts[i / 2], a = lo[i], b = lo[i + 1];
                lo[i] = a * c - b * s;
                lo[i + 1] = b * c + a * s;
            }
            if (jh < half) {
                const float c = tc[2 + i / 2], s = ts[2 + i / 2], a = hi[i], b = hi[i + 1];
                hi[i] = a * c - b * s;
                hi[i + 1] = b * c + a * s;
            }
        }
    }
}

__device__ __forceinline__ uint32_t i8x4(const float (&x)[4], float inv) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float t = fminf(fmaxf(__builtin_rintf(__fmul_rn(x[i], inv)), -127.0f), 127.0f);
        w |= ((uint32_t)(int)t & 0xFFu) << (8 * i);
    }
    return w;
}

template <int D, int MODE>
__global__ __launch_bounds__(256) void rows8_quant_kernel(const Rows8Launch a) {
    constexpr int LPR = D / 8;                  // lanes per row
    constexpr int RPP = 256 / LPR;              // rows per pass
    constexpr int NP = kTile / RPP;             // passes per tile
    __shared__ float red[2][4];
    const int tid = threadIdx.x, li = tid % LPR, lr = tid / LPR;
    const int t = blockIdx.x % a.tiles, g = blockIdx.x / a.tiles, h = blockIdx.y;
    const int64_t gstart = (int64_t)g * a.group;
    const int64_t gend = min<int64_t>(gstart + a.group, a.n);
    const int64_t row0 = gstart + (int64_t)t * kTile;
    const uint16_t *qkv = static_cast<const uint16_t *>(a.qkv);
    const int64_t rs = 3 * a.heads * D;
    const int el = 4 * li, eh = D / 2 + 4 * li;

    // Every load of the tile first (q, k, v of all its rows, and their table entries):
    // descriptors end with the group and the table, so rows past them read as zeros.
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const __amdgpu_buffer_rsrc_t rr = seq_rsrc(qkv + row0 * rs, gend > row0 ? (gend - row0) * rs * 2 : 0);
    const int64_t tbytes = MODE ? a.n * (int64_t)a.half * 4 : 0;
    const __amdgpu_buffer_rsrc_t cr = seq_rsrc(a.cos, tbytes), sr = seq_rsrc(a.sin, tbytes);
    u32x2 raw[NP][6];
    f32x4 tcv[NP], tsv[NP];
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
        const int ro = (ps * RPP + lr) * (int)rs * 2;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            raw[ps][2 * j] = __builtin_amdgcn_raw_buffer_load_b64(rr, ro + (int)((j * a.heads + h) * D + el) * 2, 0, 0);
            raw[ps][2 * j + 1] = __builtin_amdgcn_raw_buffer_load_b64(rr, ro + (int)((j * a.heads + h) * D + eh) * 2, 0, 0);
        }
        const int trow = (int)(row0 + ps * RPP + lr);
        if constexpr (MODE == 1) {
            tcv[ps] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, (trow * a.half + el) * 4, 0, 0));
            tsv[ps] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, (trow * a.half + el) * 4, 0, 0));
        } else if constexpr (MODE == 2) {
            const u32x2 c0 = __builtin_amdgcn_raw_buffer_load_b64(cr, (trow * a.half + 2 * li) * 4, 0, 0);
            const u32x2 c1 = __builtin_amdgcn_raw_buffer_load_b64(cr, (trow * a.half + D / 4 + 2 * li) * 4, 0, 0);
            const u32x2 s0 = __builtin_amdgcn_raw_buffer_load_b64(sr, (trow * a.half + 2 * li) * 4, 0, 0);
            const u32x2 s1 = __builtin_amdgcn_raw_buffer_load_b64(sr, (trow * a.half + D / 4 + 2 * li) * 4, 0, 0);
            tcv[ps] = (f32x4){__uint_as_float(c0[0]), __uint_as_float(c0[1]), __uint_as_float(c1[0]), __uint_as_float(c1[1])};
            tsv[ps] = (f32x4){__uint_as_float(s0[0]), __uint_as_float(s0[1]), __uint_as_float(s1[0]), __uint_as_float(s1[1])};
        } else {
            tcv[ps] = tsv[ps] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
    }

    float kk[NP][8];
    float kmax = 0.f, vmax = 0.f;
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
        const int64_t r = row0 + ps * RPP + lr;
        const bool ok = r < gend;
        float ql[4], qh[4], kl[4], kh[4], vl[4], vh[4];
        unpack_bf16x2(raw[ps][0][0], ql[0], ql[1]); unpack_bf16x2(raw[ps][0][1], ql[2], ql[3]);
        unpack_bf16x2(raw[ps][1][0], qh[0], qh[1]); unpack_bf16x2(raw[ps][1][1], qh[2], qh[3]);
        unpack_bf16x2(raw[ps][2][0], kl[0], kl[1]); unpack_bf16x2(raw[ps][2][1], kl[2], kl[3]);
        unpack_bf16x2(raw[ps][3][0], kh[0], kh[1]); unpack_bf16x2(raw[ps][3][1], kh[2], kh[3]);
        unpack_bf16x2(raw[ps][4][0], vl[0], vl[1]); unpack_bf16x2(raw[ps][4][1], vl[2], vl[3]);
        unpack_bf16x2(raw[ps][5][0], vh[0], vh[1]); unpack_bf16x2(raw[ps][5][1], vh[2], vh[3]);
        prep_row<D, MODE>(kl, kh, li, a.kw, tcv[ps], tsv[ps], a.half, a.eps);
        if (r < a.nq) {   // the row is a query: its own int8 scale (uniform over the LPR lanes)
            prep_row<D, MODE>(ql, qh, li, a.qw, tcv[ps], tsv[ps], a.half, a.eps);
            float qm = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) qm = fmaxf(qm, fmaxf(fabsf(ql[i]), fabsf(qh[i])));
            qm = max_lanes<LPR>(qm);
            const float s = qm > 0.f ? __fdiv_rn(qm, 127.0f) : 1.0f;
            const float inv = __fdiv_rn(1.0f, s);
            if (ok) {
                int8_t *dst = a.q8 + (r * a.heads + h) * D;
                *reinterpret_cast<uint32_t *>(dst + el) = i8x4(ql, inv);
                *reinterpret_cast<uint32_t *>(dst + eh) = i8x4(qh, inv);
                if (li == 0) a.sq[r * a.heads + h] = s;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kk[ps][i] = kl[i];
            kk[ps][4 + i] = kh[i];
            kmax = fmaxf(kmax, fmaxf(fabsf(kl[i]), fabsf(kh[i])));
            vmax = fmaxf(vmax, fmaxf(fabsf(vl[i]), fabsf(vh[i])));
        }
    }
    kmax = max_lanes<64>(kmax);
    vmax = max_lanes<64>(vmax);
    if (tid % 64 == 0) {
        red[0][tid / 64] = kmax;
        red[1][tid / 64] = vmax;
    }
    __syncthreads();
    kmax = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    vmax = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    const float sk = kmax > 0.f ? __fdiv_rn(kmax, 127.0f) : 1.0f;
    const float kinv = __fdiv_rn(1.0f, sk);
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
        const int64_t r = row0 + ps * RPP + lr;
        if (r < gend) {
            int8_t *dst = a.k8 + (r * a.heads + h) * D;
            const float lo4[4] = {kk[ps][0], kk[ps][1], kk[ps][2], kk[ps][3]};
            const float hi4[4] = {kk[ps][4], kk[ps][5], kk[ps][6], kk[ps][7]};
            *reinterpret_cast<uint32_t *>(dst + el) = i8x4(lo4, kinv);
            *reinterpret_cast<uint32_t *>(dst + eh) = i8x4(hi4, kinv);
        }
    }
    if (tid == 0) {
        a.sk[((int64_t)g * a.tiles + t) * a.heads + h] = sk;
        a.vmax[((int64_t)g * a.tiles + t) * a.heads + h] = vmax;    // the tile's amax of v
    }
}

// Position p = 32 g + b of a tile holds this key of the tile.
__device__ __forceinline__ int tile_key(int p) {
    const int g = p / 32, b = p % 32;
    return 32 * (b / 16) + 8 * ((b % 16) / 4) + 4 * g + (b % 4);
}

template <int D>
__global__ __launch_bounds__(256) void rows8_vt_kernel(const Rows8Launch a) {
    __shared__ float vs[kTile][D + 1];
    const int tid = threadIdx.x;
    const int t = blockIdx.x % a.tiles, g = blockIdx.x / a.tiles, h = blockIdx.y;
    const int64_t gstart = (int64_t)g * a.group;
    const int64_t gend = min<int64_t>(gstart + a.group, a.n);
    const int64_t row0 = gstart + (int64_t)t * kTile;
    const uint16_t *qkv = static_cast<const uint16_t *>(a.qkv);
    const int64_t rs = 3 * a.heads * D;
    // The group's amax of v is the largest of its tiles' (written by the quantizing
    // kernel): the threads read them side by side, reduced over the block below.
    __shared__ float red[4];
    float amax = 0.f;
    for (int tt = tid; tt < a.tiles; tt += 256) amax = fmaxf(amax, a.vmax[((int64_t)g * a.tiles + tt) * a.heads + h]);
    for (int idx = tid; idx < kTile * (D / 8); idx += 256) {     // 16-byte loads: 8 values each
        const int i = idx / (D / 8), e0 = 8 * (idx % (D / 8));
        const int64_t r = row0 + i;
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (r < gend) {
            const uint4 u = *reinterpret_cast<const uint4 *>(qkv + r * rs + (int64_t)(2 * a.heads + h) * D + e0);
            unpack_bf16x2(u.x, x[0], x[1]);
            unpack_bf16x2(u.y, x[2], x[3]);
            unpack_bf16x2(u.z, x[4], x[5]);
            unpack_bf16x2(u.w, x[6], x[7]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) vs[i][e0 + j] = x[j];
    }
    amax = max_lanes<64>(amax);
    if (tid % 64 == 0) red[tid / 64] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    const float inv = __fdiv_rn(1.0f, s);
    uint8_t *tile = a.v8t + (((int64_t)g * a.tiles + t) * a.heads + h) * D * kTile;
    for (int idx = tid; idx < D * 2; idx += 256) {
        const int e = idx / 2, part = idx % 2;     // d row e, positions 32 part .. + 31
        uint32_t wv[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = __fmul_rn(vs[tile_key(32 * part + 4 * w + j)][e], inv);
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], pk, true);
            wv[w] = (uint32_t)pk;
        }
        uint4 *dst = reinterpret_cast<uint4 *>(tile + e * kTile + 32 * part);
        dst[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        dst[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
    }
    if (t == 0 && tid == 0) a.sv[(int64_t)g * a.heads + h] = s;
}

// ------------------------------------------------------------------------ attention

template <int D>
struct Geo8 {
    static constexpr int kKPitch = D + 16;                 // int8 K row + one pad slot
    static constexpr int kVPitch = kTile + 16;             // E4M3 V^T row (64 keys) + pad
    static constexpr int kKSlots = kKPitch / 16, kVSlots = kVPitch / 16;
    static constexpr int kKBytes = kTile * kKPitch, kVBytes = D * kVPitch;
    static constexpr int kBuf = kKBytes + kVBytes;
    static constexpr int kKLoads = kTile * kKSlots / 64, kVLoads = D * kVSlots / 64;
    static constexpr int kLoads = kKLoads + kVLoads;
    static constexpr int kPerWave = (kLoads + 3) / 4;
    static_assert(kTile * kKSlots % 64 == 0 && D * kVSlots % 64 == 0, "whole 64-lane loads");
};

// The occupancy hint caps the register budget per wave at 256 (d = 128) or 128: with a
// larger budget the compiler keeps the products' results in accumulation registers and
// copies every score and every rescaled output value through them (about four in ten of
// the tile loop's vector instructions, on a loop bound by its vector instructions).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : 4))) void attn8_kernel(const Rows8Launch a) {
    typedef Geo8<D> G;
    constexpr int NC = D / 32;       // k steps of S^T (32 bytes each)
    constexpr int NDB = D / 32;      // 32-wide d blocks of the output
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * G::kBuf];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
    const int n = lane % 32, g = lane / 32;
    // Blocks are dealt to the XCDs round robin: give each XCD a run of consecutive
    // (query tile, head) indices, so the query tiles of a head share one L2.
    const unsigned nbx = gridDim.x, nb = nbx * gridDim.y, lin = blockIdx.x + blockIdx.y * nbx;
    const unsigned full = nb / kXcds * kXcds;
    const unsigned vid = lin < full ? (lin % kXcds) * (nb / kXcds) + lin / kXcds : lin;
    const int bx = (int)(vid % nbx), h = (int)(vid / nbx);
    const int qt = bx % a.qtiles, grp = bx / a.qtiles;
    const int64_t gstart = (int64_t)grp * a.group;
    const int64_t gend = min<int64_t>(gstart + a.group, a.n);
    const int len = (int)(gend - gstart);
    const int64_t qend = min<int64_t>(gend, a.nq);
    const int64_t r = gstart + (int64_t)qt * kBM + 32 * w + n;
    const bool row_ok = r < qend;
    const int ntiles = (len + kTile - 1) / kTile;
    if (gstart + (int64_t)qt * kBM >= qend) return;     // no query row in this block (block-uniform)

    // tile loads: slot s of the buffer (K slots first, then V^T slots); wave w takes loads
    // w, w + 4, ...; a pad slot repeats its row's last data chunk (never read).
    const int64_t krs = (int64_t)a.heads * D;
    const uint8_t *kbase = reinterpret_cast<const uint8_t *>(a.k8) + (gstart * a.heads + h) * D;
    int voff[G::kPerWave];
    bool isk[G::kPerWave];
#pragma unroll
    for (int t = 0; t < G::kPerWave; ++t) {
        const int ld = w + 4 * t;
        const int slot = ld * 64 + lane;
        isk[t] = ld < G::kKLoads;
        if (isk[t]) {
            const int row = slot / G::kKSlots, col = slot % G::kKSlots;
            voff[t] = (int)(row * krs + 16 * min(col, D / 16 - 1));
        } else {
            const int vs = slot - G::kKLoads * 64;
            const int row = vs / G::kVSlots, col = vs % G::kVSlots;
            voff[t] = row * kTile + 16 * min(col, kTile / 16 - 1);
        }
    }
    auto load_tile = [&](int kt, int bsel) {
        const int key0 = kt * kTile;
        const __amdgpu_buffer_rsrc_t kr = seq_rsrc(kbase + key0 * krs, ((int64_t)(len - 1 - key0) * krs + D));
        const __amdgpu_buffer_rsrc_t vr = seq_rsrc(a.v8t + (((int64_t)grp * a.tiles + kt) * a.heads + h) * D * kTile,
                                                   (int64_t)D * kTile);
        unsigned char *dst = smem + bsel * G::kBuf;
#pragma unroll
        for (int t = 0; t < G::kPerWave; ++t) {
            const int ld = w + 4 * t;
            if (ld < G::kLoads) buffer_to_lds16(isk[t] ? kr : vr, dst + ld * 1024, voff[t]);
        }
    };

    load_tile(0, 0);

    // Query fragments (B of S^T): row r, bytes 32 c + 16 g .. + 15; rows past the end read 0.
    i32x4 qf[NC];
    {
        const int64_t row0w = gstart + (int64_t)qt * kBM + 32 * w;
        const int64_t wrows = min<int64_t>(32, qend - row0w);
        const __amdgpu_buffer_rsrc_t qr = seq_rsrc(a.q8 + (row0w * a.heads + h) * D,
                                                   wrows > 0 ? ((wrows - 1) * a.heads * D + D) : 0);
#pragma unroll
        for (int c = 0; c < NC; ++c)
            qf[c] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, (int)(n * a.heads * D + 32 * c + 16 * g), 0, 0));
    }
    const float arow = row_ok ? a.sq[r * a.heads + h] * a.scale * kLog2e : 0.f;
    const float kLog2Max = 8.807354922057604f;     // log2 448
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    const int k_lane = n * G::kKPitch + 16 * g;
    const int v_lane = G::kKBytes + n * G::kVPitch + 32 * g;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = 0; kt < ntiles; ++kt) {
        const int bsel = kt & 1;
        if (kt + 1 < ntiles) load_tile(kt + 1, bsel ^ 1);
        const unsigned char *buf = smem + bsel * G::kBuf;
        i32x16 si[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) si[kb][i] = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const i32x4 ka = *reinterpret_cast<const i32x4 *>(buf + k_lane + kb * 32 * G::kKPitch + 32 * c);
                si[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qf[c], si[kb], 0, 0, 0);
            }
        // Scores in base-2 units are si * f (f >= 0), so the tile max is taken on the integers.
        const float f = arow * a.sk[((int64_t)grp * a.tiles + kt) * a.heads + h];
        const int key0 = kt * kTile;
        if (key0 + kTile > len) {          // the group's last, ragged tile (block-uniform)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (key0 + 32 * kb + 8 * (i / 4) + 4 * g + (i % 4) >= len) si[kb][i] = INT32_MIN;
        }
        int mi = si[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mi = max(mi, si[kb][i]);
        float mx = mi == INT32_MIN ? -INFINITY : (float)mi * f;
        mx = fmaxf(mx, lane_pair8(mx, g));
        const float m_new = fmaxf(m_run, mx);
        if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
            const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            m_run = m_new;
        }
        const float bias = m_run == -INFINITY ? 0.f : kLog2Max - m_run;
        i32x8 pk;
#pragma unroll
        for (int wd = 0; wd < 8; ++wd) {
            const int kb = wd / 4, i0 = 4 * (wd % 4);
            float p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // a masked key (INT32_MIN) gives 2^-huge = 0; f is finite, so no inf - inf
                p[j] = fast_exp2(fmaf((float)si[kb][i0 + j], f, bias));
                l_run += p[j];
            }
            int v = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], v, true);
            pk[wd] = v;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const unsigned char *va = buf + v_lane + db * 32 * G::kVPitch;
            const i32x4 lo = *reinterpret_cast<const i32x4 *>(va);
            const i32x4 hi = *reinterpret_cast<const i32x4 *>(va + 16);
            const i32x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pk, o[db], 0, 0, 0, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    const float l_tot = l_run + lane_pair8(l_run, g);
    if (row_ok) {
        const float sv = a.sv[(int64_t)grp * a.heads + h];
        const float mul = l_tot > 0.f ? sv / l_tot : 0.f;
        uint16_t *orow = static_cast<uint16_t *>(a.out) + (r * a.heads + h) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint2 u;
                u.x = pack_bf16x2(o[db][4 * i] * mul, o[db][4 * i + 1] * mul);
                u.y = pack_bf16x2(o[db][4 * i + 2] * mul, o[db][4 * i + 3] * mul);
                *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * i + 4 * g) = u;
            }
    }
}

template <int D>
void launch_quant_d(const Rows8Launch &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.groups * a.tiles), (unsigned)a.heads);
    if (a.prep_mode == 0)
        hipLaunchKernelGGL((rows8_quant_kernel<D, 0>), grid, dim3(256), 0, stream, a);
    else if (a.prep_mode == 1)
        hipLaunchKernelGGL((rows8_quant_kernel<D, 1>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((rows8_quant_kernel<D, 2>), grid, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((rows8_vt_kernel<D>), grid, dim3(256), 0, stream, a);
}

}  // namespace

hipError_t launch_rows8_quantize(const Rows8Launch &a, hipStream_t stream) {
    if (a.d == 64) launch_quant_d<64>(a, stream); else launch_quant_d<128>(a, stream);
    return hipGetLastError();
}

hipError_t launch_rows8_attend(const Rows8Launch &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.groups * a.qtiles), (unsigned)a.heads);
    if (a.d == 64)
        hipLaunchKernelGGL((attn8_kernel<64>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((attn8_kernel<128>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn
