// Device helpers for the bf16 kernels: vector types, bf16 <-> f32, MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (x in the low half), round to nearest even
// (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ inline uint32_t pack_bf16(float x, float y) {
  bf16x2 r = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(uint32_t, r);
}

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).
// Operand layout (lane l, slot s = 0..7): A[m = l%32][k = 8*(l/32) + s],
// B[k = 8*(l/32) + s][n = l%32].  Result register i of lane l holds
// D[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ inline f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Reductions across the two 32-lane halves of a wavefront (lanes l and l^32)
// with v_permlane32_swap: swap(x, x) yields the pair (x[l], x[l^32]) in every lane.
__device__ inline float halves_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float halves_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

}  // namespace gattn
