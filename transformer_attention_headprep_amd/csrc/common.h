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

}  // namespace attn
