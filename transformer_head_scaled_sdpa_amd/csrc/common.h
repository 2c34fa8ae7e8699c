// Shared device-side definitions of the gfx950 attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

typedef uint16_t bf16_t;  // raw bfloat16 storage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// log2(e): softmax exponentials are evaluated as exp2 of log2(e)-scaled scores.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = static_cast<__bf16>(lo);
    v[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second;
// given the same value twice, element 0 of the result holds x[l % 32] and
// element 1 holds x[l % 32 + 32] in every lane.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mha
