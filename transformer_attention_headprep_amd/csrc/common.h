// common.h -- device helpers shared by the HIP kernels of libattn (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 1 / ln 2: scores are kept in base-2 units so the softmax uses exp2.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round two f32 to bf16, nearest even (v_cvt_pk_bf16_f32), packed low = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 h = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// Unpack the two bf16 of a 32-bit word to f32 (low half first).
__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float &lo, float &hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xFFFF0000u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Butterfly reductions over `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float sum_lanes(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

template <int WIDTH>
__device__ __forceinline__ float max_lanes(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Buffer descriptor over `bytes` bytes from `base` (raw, untyped; reads past the end
// return zero).  The arguments must be wave-uniform; readfirstlane keeps it in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const void *base, int64_t bytes) {
    const int n = bytes > 0 ? (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF) : 0;
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *sbase = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(sbase, (short)0, __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

// Cache-policy bits of a buffer access: kStream (nt, non-temporal) marks data read once,
// so that streaming it does not push out lines the caches hold for reuse -- or that are
// still waiting to be written back.
constexpr int kStream = 2;

// XCDs (accelerator complex dies, each with its own L2) of the chip; a launch deals its
// blocks to them round robin.
constexpr int kXcds = 8;

// 16 bytes per lane from a buffer straight into LDS: lane L writes lds + 16 L (policy:
// 0 or kStream).
template <int POLICY = 0>
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rsrc, void *lds, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds, 16, voffset,
                                             0, 0, POLICY);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element i % 4 of
// the four 4 x 16-bit vectors addressed by lanes 4 r + i / 4, r = 0..3 (in order r).
__device__ __forceinline__ i16x4 lds_read_tr16(const void *lds) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(lds));
}

// A paged KV pool seen by a kernel: row `key` of sequence b is pool row
// (pages[b max_pages + key >> shift] << shift) + (key & (2^shift - 1)).  pages == NULL:
// no pool.  A page id outside [0, num_pages) sets `bad` and maps to page 0.
struct PageMap {
    const int32_t *pages;
    int shift, max_pages, num_pages;
};
__device__ __forceinline__ int64_t pool_row(const PageMap &m, int b, int64_t key, bool &bad) {
    int id = m.pages[(int64_t)b * m.max_pages + (key >> m.shift)];
    if ((unsigned)id >= (unsigned)m.num_pages) {
        bad = true;
        id = 0;
    }
    return ((int64_t)id << m.shift) + (key & (((int64_t)1 << m.shift) - 1));
}

// Wait until at most n vector-memory loads of this wave are outstanding (vmcnt only).
#define ATTN_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

// Four transposing LDS reads (as lds_read_tr16) that complete before this returns.  Next
// to loads that write LDS directly, the compiler waits for all of them before an LDS
// read whenever it cannot tell that the read touches none of their bytes (always for
// the transposing builtin, and for plain reads in a loop that rotates buffers); these
// forms leave those waits to the caller.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void lds_read_tr16_x4(i16x4 &a0, i16x4 &a1, i16x4 &a2, i16x4 &a3, uint32_t o0, uint32_t o1,
                                                 uint32_t o2, uint32_t o3) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
        : "v"(o0), "v"(o1), "v"(o2), "v"(o3)
        : "memory");
}

// Two 16-byte LDS reads that complete before this returns (the same reason as above).
__device__ __forceinline__ void lds_read_b128_x2(bf16x8 &a0, bf16x8 &a1, uint32_t o0, uint32_t o1) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1)
        : "v"(o0), "v"(o1)
        : "memory");
}

// Workgroup barrier that orders LDS accesses only: this wave's LDS reads and writes
// complete, then the barrier.  __syncthreads() (and a release fence on LDS alone) also
// waits for every load of this wave that writes LDS directly, loads issued for later
// tiles included; such loads are waited for explicitly (ATTN_WAIT_VMCNT) before this.
// The memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace attn
