// kvq.hip -- the quantised KV cache: its coding pass and the decode that reads it.
//
// Keys and values kept in 8, 4 or 2 bits, each head of each token coded over the range
// that returns it with the least squared error (compute guide "Tensors, GPU kernels and
// AI models", Step 5: Run a language model).  A coded head is d codes c in [0, 2^bits)
// and a pair (lo, step): it returns lo + step c.  The range is chosen among 24 candidates
// centred on (min + max)/2 with half-widths (max - min)/2 (32 - k)/32; every operation
// that decides a code runs in f32 in a fixed order (correctly rounded division, no
// contraction), and the squared error of a candidate is summed in f64.
//
// Layout (head-major, so a block of the decode streams one kv head's rows):
//   codes  [batch, heads, capacity, d bits / 8] bytes; each 32-bit little-endian word
//          holds 32 / bits consecutive codes, code j at bit (j mod 2) 16 + (j / 2) bits:
//          even codes in the low half-word, odd ones in the high half-word, so one mask
//          puts a pair of adjacent codes into the two 16-bit lanes of a register.
//   params [batch, heads, capacity, 2] f32 (lo, step).
//
// The decode (decode_q_kernel) is decode_bf16_kernel's design with the cache rows
// turned into bf16 matrix-core operands as they arrive (keys straight from registers:
// lane (n, kk) loads row n's codes of dims kk D/4 .., the A fragments of its products, and
// q's fragments take the same dims; values through LDS for the transposing reads):
//   - 8 bits: a code c becomes the bf16 c (exact: integers below 256 have 8 bits);
//   - 4 and 2 bits: a pair of codes becomes the bf16 pair 128 + c (0x4300 | c, one
//     mask-and-or per pair), i.e. an offset M = 128 that is taken out again below.
//   With the operand value u = M + c, a key's score is step q.u + (lo - M step) sum(q):
//   the products run on the matrix cores over the codes, and each key's (lo, step)
//   enters as one fused multiply-add on the lane that holds the key's score.  On the
//   value side a weight p becomes p step (as a bf16 high part plus a bf16 remainder, two
//   MFMAs, since u carries the offset M), and sum_j p_j (lo_j - M step_j) is added to
//   every output value of the head at the end.
#include "decode_common.h"

namespace attn {
namespace {

// --------------------------------------------------------------------------- coding

template <bool BF16, int D, int BITS>
__global__ __launch_bounds__(256) void kv_quantize_kernel(const KvQuantLaunch a, int64_t units) {
    constexpr int LPU = D / 8;                  // lanes per unit, 8 values each
    constexpr int UPB = 256 / LPU;              // units per block
    constexpr int TOP = (1 << BITS) - 1;
    constexpr int RB = D * BITS / 8;            // bytes of one coded head
    const int li = threadIdx.x % LPU;
    const int64_t unit = (int64_t)blockIdx.x * UPB + threadIdx.x / LPU;
    const bool valid = unit < units;
    const int64_t uu = valid ? unit : 0;
    const int64_t h = uu % a.heads, row = uu / a.heads, t = row % a.seq, bb = row / a.seq;

    float x[8];
    const int64_t off = bb * a.seq * a.rs + t * a.rs + h * D + 8 * li;
    if constexpr (BF16) {
        const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + off);
        unpack_bf16x2(w.x, x[0], x[1]);
        unpack_bf16x2(w.y, x[2], x[3]);
        unpack_bf16x2(w.z, x[4], x[5]);
        unpack_bf16x2(w.w, x[6], x[7]);
    } else {
        const float4 u0 = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + off);
        const float4 u1 = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + off + 4);
        x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
        x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
    }
#pragma unroll
    for (int o = LPU / 2; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, 64));
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    }
    const float centre = __fmul_rn(__fadd_rn(mn, mx), 0.5f);
    const float r = __fmul_rn(__fsub_rn(mx, mn), 0.5f);
    const bool flat = !(r > 1e-30f);

    // The candidate ranges, in the order and precision the codes are defined by.
    auto candidate = [&](int k, float &lo, float &st, float &inv) {
        const float hw = __fmul_rn(r, (float)(32 - k) * 0.03125f);
        lo = __fsub_rn(centre, hw);
        st = __fdiv_rn(__fadd_rn(hw, hw), (float)TOP);
        inv = __fdiv_rn(1.0f, st);
    };
    auto code = [&](float v, float lo, float inv) {
        return fminf(fmaxf(__builtin_rintf(__fmul_rn(__fsub_rn(v, lo), inv)), 0.0f), (float)TOP);
    };
    int best_k = 0;
    if (!flat) {
        double best = INFINITY;
        for (int k = 0; k < 24; ++k) {
            float lo, st, inv;
            candidate(k, lo, st, inv);
            double sse = 0.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double back = __dadd_rn((double)lo, __dmul_rn((double)st, (double)code(x[i], lo, inv)));
                const double err = __dsub_rn((double)x[i], back);
                sse = __dadd_rn(sse, __dmul_rn(err, err));
            }
#pragma unroll
            for (int o = LPU / 2; o > 0; o >>= 1) sse += __shfl_xor(sse, o, 64);
            if (sse < best) {
                best = sse;
                best_k = k;
            }
        }
    }
    float lo = mn, st = 0.f, inv = 0.f;
    if (!flat) candidate(best_k, lo, st, inv);
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = flat ? 0u : (uint32_t)code(x[i], lo, inv);

    const int64_t drow = (bb * a.heads + h) * a.capacity + a.row0 + t;   // cache row of this unit
    uint8_t *dst = a.codes + drow * RB;
    if constexpr (BITS == 8) {
        // two words of 4 codes: j at bit (j % 2) 16 + (j / 2) 8
        uint2 wv;
        wv.x = c[0] | (c[2] << 8) | (c[1] << 16) | (c[3] << 24);
        wv.y = c[4] | (c[6] << 8) | (c[5] << 16) | (c[7] << 24);
        if (valid) *reinterpret_cast<uint2 *>(dst + 8 * li) = wv;
    } else if constexpr (BITS == 4) {
        uint32_t wv = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) wv |= c[j] << ((j % 2) * 16 + (j / 2) * 4);
        if (valid) *reinterpret_cast<uint32_t *>(dst + 4 * li) = wv;
    } else {
        // a word of 16 codes spans this lane (codes 0..7 of it if li is even) and its pair
        uint32_t part = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = (li % 2) * 8 + i;
            part |= c[i] << ((j % 2) * 16 + (j / 2) * 2);
        }
        const uint32_t wv = part | __shfl_xor(part, 1, 64);
        if (valid && li % 2 == 0) *reinterpret_cast<uint32_t *>(dst + 4 * (li / 2)) = wv;
    }
    if (valid && li == 0) *reinterpret_cast<float2 *>(a.params + drow * 2) = make_float2(lo, st);
}

template <bool BF16, int D>
void launch_quant_d(const KvQuantLaunch &a, int64_t units, hipStream_t stream) {
    constexpr int UPB = 256 / (D / 8);
    const dim3 grid((unsigned)((units + UPB - 1) / UPB));
    if (a.bits == 8)
        hipLaunchKernelGGL((kv_quantize_kernel<BF16, D, 8>), grid, dim3(256), 0, stream, a, units);
    else if (a.bits == 4)
        hipLaunchKernelGGL((kv_quantize_kernel<BF16, D, 4>), grid, dim3(256), 0, stream, a, units);
    else
        hipLaunchKernelGGL((kv_quantize_kernel<BF16, D, 2>), grid, dim3(256), 0, stream, a, units);
}

// --------------------------------------------------------------------------- decode

// Loads of one chunk (16 rows) of a coded tensor: every lane reads LB bytes, NL times.
template <int D, int BITS>
struct QGeo {
    static constexpr int kRB = D * BITS / 8;                 // bytes of one coded row
    static constexpr int kLB = kRB >= 64 ? 16 : kRB / 4;     // bytes per lane per load
    static constexpr int kNL = kChunk * kRB / (64 * kLB);    // loads per lane per chunk
    static constexpr int kWords = kLB / 4;
    static constexpr int kCodes = kLB * 8 / BITS;            // codes per lane per load
    static constexpr int kM = BITS == 8 ? 0 : 128;           // operand offset (u = M + c)
    static_assert(kChunk * kRB == 64 * kLB * kNL, "whole loads");
    static_assert(kCodes % 8 == 0, "whole 16-byte bf16 slots");
};

// LB bytes a lane of a coded tensor, streamed (read once).
template <int LB>
__device__ __forceinline__ void load_words(uint32_t *w, __amdgpu_buffer_rsrc_t rs, int off) {
    if constexpr (LB == 16) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kStream);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    } else if constexpr (LB == 8) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kStream);
        w[0] = v[0]; w[1] = v[1];
    } else {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kStream);
    }
}

// The bf16 operand pairs of word w (32 / BITS consecutive codes): pair i holds codes
// 2i and 2i + 1 as bf16 values M + c.
template <int BITS>
__device__ __forceinline__ void word_pairs(uint32_t w, uint32_t *out, uint32_t bias = 0x43004300u) {
    if constexpr (BITS == 8) {
        // j = 0, 1 at bytes 0, 2; j = 2, 3 at bytes 1, 3.  Integers below 256 are exact
        // in bf16: the high half of their f32.
        const float f0 = (float)(w & 0xFFu), f1 = (float)((w >> 16) & 0xFFu);
        const float f2 = (float)((w >> 8) & 0xFFu), f3 = (float)(w >> 24);
        out[0] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
        out[1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
    } else {
        constexpr uint32_t mask = ((1u << BITS) - 1) * 0x00010001u;
#pragma unroll
        for (int i = 0; i < 16 / BITS; ++i) out[i] = ((w >> (BITS * i)) & mask) | bias;
    }
}

// Store a lane's loaded codes of one chunk as bf16 operands into the rows of the chunk's
// K (IS_K) or V buffer, in the bf16 decode's swizzled layout.
template <int D, int BITS, bool IS_K>
__device__ __forceinline__ void stage_codes(unsigned char *buf, const uint32_t (*words)[QGeo<D, BITS>::kWords], int lane,
                                            uint32_t bias = 0x43004300u) {
    typedef QGeo<D, BITS> Q;
    typedef DecGeo<D> G;
#pragma unroll
    for (int i = 0; i < Q::kNL; ++i) {
        const int o = (64 * i + lane) * Q::kLB;
        const int row = o / Q::kRB;
        const int d0 = (o % Q::kRB) * 8 / BITS;
        uint32_t pr[Q::kCodes / 2];
#pragma unroll
        for (int wd = 0; wd < Q::kWords; ++wd) word_pairs<BITS>(words[i][wd], pr + wd * (16 / BITS), bias);
#pragma unroll
        for (int sl = 0; sl < Q::kCodes / 8; ++sl) {
            const int slot = d0 / 8 + sl;
            const int phys = IS_K ? kslot<D>(row, slot) : vslot<D>(row, slot);
            const u32x4 v4 = {pr[4 * sl], pr[4 * sl + 1], pr[4 * sl + 2], pr[4 * sl + 3]};
            *reinterpret_cast<u32x4 *>(buf + row * G::kRow + 16 * phys) = v4;
        }
    }
}

// x, held in a vector register (the compiler cannot fold it back into a literal).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Lane (lane & ~3) + i's value: the i-th of the lane's quad (DPP quad permute).
__device__ __forceinline__ uint32_t quad_lane(uint32_t v, int i) {
    switch (i) {
        case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, false);
        case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, false);
        case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, false);
        default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, false);
    }
}

// At d = 128 the occupancy hint asks for no more than two waves per SIMD: a higher one
// caps the vector registers at 128, and the compiler then parks the excess in
// accumulation registers (or scratch) and copies it back and forth inside the chunk loop
// (about a fifth of the loop's vector instructions at 4/4).  Without the cap the 4- and
// 2-bit kernels need ~150 registers, so three waves per SIMD still fit; 8-bit ~180 (two).
template <int D, int GB, int KB, int VB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : (GB <= 4 ? 4 : 3)))) void decode_q_kernel(const DecodeParams p) {
    typedef DecGeo<D> G;
    typedef QGeo<D, KB> GK;
    typedef QGeo<D, VB> GV;
    constexpr int kTiles = kWaves * 2 * G::kBuf;
    constexpr int kQBytes = 2 * GB * D * 4 + 4 * (kThreads / 64);
    constexpr int kOBytes = kWaves * GB * D * 4 + 2 * kWaves * GB * 4;
    static_assert(kQBytes <= kTiles && kOBytes <= kTiles, "prologue and merge fit the tile region");
    constexpr int kQFrag = 2 * G::kKMfma * 64 * 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kTiles + kQFrag];
    __shared__ int s_page_bad;                 // some wave met a page id outside the pool

    const int tid = threadIdx.x, lane = tid % 64;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    if (tid == 0) s_page_bad = 0;              // seen by all after the prologue's barriers
    const BlockCoord bc = block_coord(p);
    const int b = bc.b, split = bc.split;
    const int h0 = bc.kvh * p.group + bc.grp * GB;
    const int nh = min(GB, p.group - bc.grp * GB);

    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.max_len ? (int)p.max_len : len);
    const int start = split * (int)p.per_split;
    const int end = min(len, start + (int)p.per_split);

    // Codes and (lo, step) pairs are head-major in each unit (a sequence's cache, or a
    // pool page): row r of kv head kvh of unit u is coded row (u hkv + kvh) rows + r.
    const int64_t urows = unit_rows(p);
    bool page_bad = false;
    auto coded_row = [&](int key0) -> int64_t {
        const CacheSlot cs = key0 < end ? cache_slot(p, b, key0, page_bad) : CacheSlot{0, 0};
        return ((int64_t)cs.unit * p.hkv + bc.kvh) * urows + cs.row;
    };
    unsigned char *kbuf = smem + w * 2 * G::kBuf;
    unsigned char *vbuf = kbuf + G::kBuf;

    const int first = start + kChunk * w;
    const int nch = end > first ? (end - first + kChunk * kWaves - 1) / (kChunk * kWaves) : 0;
    const int n = lane % 16, kk = lane / 16;

    // A chunk in registers: the lane's code words and the (lo, step) pairs of key
    // 4 kk + n % 4 (the other keys of the lane's four come from its quad, by DPP).
    // Key codes: lane (n, kk) holds row n's codes of dims kk D/4 .. (kk+1) D/4 - 1, the A
    // fragments of its kKMfma products straight from registers (q's fragments take the
    // same dims); values go through LDS for the transposing reads.
    constexpr int kKW = D * KB / 128;          // words of key codes per lane (D/4 codes)
    struct Regs {
        uint32_t k[kKW];
        uint32_t v[GV::kNL][GV::kWords];
        uint32_t kp[2], vp[2];
    };
    // Chunk j: descriptors end at the last valid row (rows past it read as zeros).
    // A chunk's 16 rows lie in one unit (pages hold a multiple of 16 rows).
    auto issue = [&](int j, Regs &r) {
        const int key0 = first + kChunk * kWaves * j;
        const int rows = min(kChunk, end - key0);
        const int64_t cr = coded_row(key0);
        const __amdgpu_buffer_rsrc_t kr = seq_rsrc(static_cast<const uint8_t *>(p.k) + cr * GK::kRB, (int64_t)rows * GK::kRB);
        const __amdgpu_buffer_rsrc_t vr = seq_rsrc(static_cast<const uint8_t *>(p.v) + cr * GV::kRB, (int64_t)rows * GV::kRB);
        const __amdgpu_buffer_rsrc_t kpr = seq_rsrc(p.kpar + cr * 2, (int64_t)rows * 8);
        const __amdgpu_buffer_rsrc_t vpr = seq_rsrc(p.vpar + cr * 2, (int64_t)rows * 8);
        {
            const int ko = n * GK::kRB + kk * (GK::kRB / 4);
            if constexpr (kKW == 8) {
                load_words<16>(r.k, kr, ko);
                load_words<16>(r.k + 4, kr, ko + 16);
            } else {
                load_words<kKW * 4>(r.k, kr, ko);
            }
        }
#pragma unroll
        for (int i = 0; i < GV::kNL; ++i) load_words<GV::kLB>(r.v[i], vr, (64 * i + lane) * GV::kLB);
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const int pofs = 8 * (4 * kk + n % 4);
        const u32x2 kp2 = __builtin_amdgcn_raw_buffer_load_b64(kpr, pofs, 0, kStream);
        const u32x2 vp2 = __builtin_amdgcn_raw_buffer_load_b64(vpr, pofs, 0, kStream);
        r.kp[0] = kp2[0]; r.kp[1] = kp2[1];
        r.vp[0] = vp2[0]; r.vp[1] = vp2[1];
    };

    // Four chunks in registers: two in flight while two are computed.
    Regs ra, rb, ra2, rb2;
    issue(0, ra);
    issue(1, rb);

    float (*qs)[D] = reinterpret_cast<float (*)[D]>(smem);
    float (*qh)[D] = reinterpret_cast<float (*)[D]>(smem + GB * D * 4);
    q_prologue<true, D, GB>(p, b, h0, nh, qs, qh, reinterpret_cast<float *>(smem + 2 * GB * D * 4));

    // q as a bf16 high part and a bf16 remainder (B fragments of S^T, as in the bf16
    // decode), and sq = the sum of exactly those values for head n (the scores' offset).
    u32x4 *qf = reinterpret_cast<u32x4 *>(smem + kTiles);
    if (w == 0) {
#pragma unroll
        for (int c = 0; c < G::kKMfma; ++c) {
            u32x4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
            if (n < nh) {
                const float *src = &qh[n][kk * (D / 4) + 8 * c];
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
    float sq = 0.f;
    if (n < nh) {
        for (int e = (D / 4) * kk; e < (D / 4) * (kk + 1); e += 2) {
            const uint32_t hv = pack_bf16x2(qh[n][e], qh[n][e + 1]);
            float ha, hb, la, lb;
            unpack_bf16x2(hv, ha, hb);
            unpack_bf16x2(pack_bf16x2(qh[n][e] - ha, qh[n][e + 1] - hb), la, lb);
            sq += (ha + la) + (hb + lb);
        }
    }
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    __syncthreads();     // q rows are dead: the LDS now holds K and V chunks

    f32x4 acc[G::kNT];
#pragma unroll
    for (int t = 0; t < G::kNT; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, thr = -INFINITY, l_lane = 0.f, b_lane = 0.f;

    // Two of this wave's chunks (j, j + 1) per step: two independent score chains, one
    // maximum over both, and their P V products interleaved per output block.  Chunk j's
    // values are staged in vbuf, chunk j + 1's in kbuf (keys never go through LDS here).
    auto compute2 = [&](int j, const Regs &ra_, const Regs &rb_) {
        const int key0a = first + kChunk * kWaves * j;
        const int key0b = key0a + kChunk * kWaves;
        // (the bf16 bias 128 of each code pair held in a vector register: an and-or then
        // takes one instruction, where two literal operands would need two)
        const uint32_t bias = in_vgpr(0x43004300u);
        stage_codes<D, VB, false>(vbuf, ra_.v, lane, bias);
        stage_codes<D, VB, false>(kbuf, rb_.v, lane, bias);
        uint32_t kpa[D / 8], kpb[D / 8];
#pragma unroll
        for (int wd = 0; wd < kKW; ++wd) {
            word_pairs<KB>(ra_.k[wd], kpa + wd * (16 / KB), bias);
            word_pairs<KB>(rb_.k[wd], kpb + wd * (16 / KB), bias);
        }
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < G::kKMfma; ++c) {
            const u32x4 ka4 = {kpa[4 * c], kpa[4 * c + 1], kpa[4 * c + 2], kpa[4 * c + 3]};
            const u32x4 kb4 = {kpb[4 * c], kpb[4 * c + 1], kpb[4 * c + 2], kpb[4 * c + 3]};
            const bf16x8 qh8 = __builtin_bit_cast(bf16x8, qf[64 * (2 * c) + lane]);
            const bf16x8 ql8 = __builtin_bit_cast(bf16x8, qf[64 * (2 * c + 1) + lane]);
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka4), qh8, sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb4), qh8, sb, 0, 0, 0);
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka4), ql8, sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb4), ql8, sb, 0, 0, 0);
        }
        // The keys' ranges: score = step q.u + (lo - M step) sq.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float kla = __uint_as_float(quad_lane(ra_.kp[0], i)), ksa = __uint_as_float(quad_lane(ra_.kp[1], i));
            const float klb = __uint_as_float(quad_lane(rb_.kp[0], i)), ksb = __uint_as_float(quad_lane(rb_.kp[1], i));
            sa[i] = fmaf(ksa, sa[i], (kla - (float)GK::kM * ksa) * sq);
            sb[i] = fmaf(ksb, sb[i], (klb - (float)GK::kM * ksb) * sq);
        }
        if (key0b + kChunk > end) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (key0a + 4 * kk + i >= end) sa[i] = -INFINITY;
                if (key0b + 4 * kk + i >= end) sb[i] = -INFINITY;
            }
        }
        const float mx = fmaxf(fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])), fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3])));
        if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
            float mh = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mh = fmaxf(mh, __shfl_xor(mh, 32, 64));
            const float m_new = fmaxf(m_run, mh * p.C);
            const float alpha = fast_exp2(m_run - m_new);
            l_lane *= alpha;
            b_lane *= alpha;
#pragma unroll
            for (int t = 0; t < G::kNT; ++t) acc[t] *= alpha;
            m_run = m_new;
            thr = (m_run + kRaiseAbove) / p.C;
        }
        // weights, as bf16 high parts and remainders of p step (chunk a, then b)
        auto weights = [&](const f32x4 &sc4, const Regs &r, i16x4 &pfh, i16x4 &pfl) __attribute__((always_inline)) {
            float pr[4], ps[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[i] = fast_exp2(fmaf(sc4[i], p.C, -m_run));
                const float vlo = __uint_as_float(quad_lane(r.vp[0], i)), vst = __uint_as_float(quad_lane(r.vp[1], i));
                ps[i] = pr[i] * vst;
                b_lane = fmaf(pr[i], vlo - (float)GV::kM * vst, b_lane);
            }
            l_lane += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            const uint32_t h01 = pack_bf16x2(ps[0], ps[1]), h23 = pack_bf16x2(ps[2], ps[3]);
            float a0, a1, a2, a3;
            unpack_bf16x2(h01, a0, a1);
            unpack_bf16x2(h23, a2, a3);
            const uint32_t l01 = pack_bf16x2(ps[0] - a0, ps[1] - a1), l23 = pack_bf16x2(ps[2] - a2, ps[3] - a3);
            pfh = __builtin_bit_cast(i16x4, make_uint2(h01, h23));
            pfl = __builtin_bit_cast(i16x4, make_uint2(l01, l23));
        };
        i16x4 pha, pla, phb, plb;
        weights(sa, ra_, pha, pla);
        weights(sb, rb_, phb, plb);
        const int vkey = 4 * kk + (lane % 16) / 4, q = lane % 4;
#pragma unroll
        for (int t = 0; t < G::kNT; ++t) {
            const int vo = vkey * G::kRow + 16 * vslot<D>(vkey, 2 * t + q / 2) + 8 * (q % 2);
            const i16x4 aa = lds_read_tr16(vbuf + vo);
            const i16x4 ab = lds_read_tr16(kbuf + vo);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aa, pha, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aa, pla, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ab, phb, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ab, plb, acc[t], 0, 0, 0);
        }
    };

    for (int j = 0; j < nch; j += 4) {
        issue(j + 2, ra2);
        issue(j + 3, rb2);
        compute2(j, ra, rb);
        if (j + 2 >= nch) break;
        issue(j + 4, ra);
        issue(j + 5, rb);
        compute2(j + 2, ra2, rb2);
    }

    // The ranges' offsets of the values: every output value of head n gains sum p (lo - M step).
    float l_head = l_lane + __shfl_xor(l_lane, 16, 64);
    l_head += __shfl_xor(l_head, 32, 64);
    float b_head = b_lane + __shfl_xor(b_lane, 16, 64);
    b_head += __shfl_xor(b_head, 32, 64);
#pragma unroll
    for (int t = 0; t < G::kNT; ++t) acc[t] += b_head;
    if (page_bad && lane == 0) s_page_bad = 1;
    __syncthreads();
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

template <int D, int KB, int VB>
void launch_q_gb(const DecodeParams &p, int gb, hipStream_t stream) {
    const dim3 grid((unsigned)(p.hkv * p.ngroups), (unsigned)p.splits, (unsigned)p.batch);
    switch (gb) {
        case 1: hipLaunchKernelGGL((decode_q_kernel<D, 1, KB, VB>), grid, dim3(kThreads), 0, stream, p); break;
        case 2: hipLaunchKernelGGL((decode_q_kernel<D, 2, KB, VB>), grid, dim3(kThreads), 0, stream, p); break;
        case 4: hipLaunchKernelGGL((decode_q_kernel<D, 4, KB, VB>), grid, dim3(kThreads), 0, stream, p); break;
        default: hipLaunchKernelGGL((decode_q_kernel<D, 8, KB, VB>), grid, dim3(kThreads), 0, stream, p); break;
    }
}

template <int D>
void launch_q_bits(const DecodeParams &p, int gb, int kb, int vb, hipStream_t stream) {
    if (kb == 8 && vb == 8) launch_q_gb<D, 8, 8>(p, gb, stream);
    else if (kb == 4 && vb == 4) launch_q_gb<D, 4, 4>(p, gb, stream);
    else if (kb == 4 && vb == 2) launch_q_gb<D, 4, 2>(p, gb, stream);
    else launch_q_gb<D, 2, 2>(p, gb, stream);
}

}  // namespace

hipError_t launch_kv_quantize(const KvQuantLaunch &a, hipStream_t stream) {
    const int64_t units = a.batch * a.seq * a.heads;
    if (units == 0) return hipSuccess;
    if (a.d == 64) {
        if (a.bf16) launch_quant_d<true, 64>(a, units, stream); else launch_quant_d<false, 64>(a, units, stream);
    } else {
        if (a.bf16) launch_quant_d<true, 128>(a, units, stream); else launch_quant_d<false, 128>(a, units, stream);
    }
    return hipGetLastError();
}

hipError_t launch_decode_q(const DecodeLaunch &a, hipStream_t stream) {
    const DecodeParams p = make_decode_params(a);
    const int gb = (int)decode_heads_per_block(a.hq, a.hkv);
    if (a.d == 64) launch_q_bits<64>(p, gb, a.kbits, a.vbits, stream);
    else launch_q_bits<128>(p, gb, a.kbits, a.vbits, stream);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_decode_merge(a, stream);
}

}  // namespace attn
