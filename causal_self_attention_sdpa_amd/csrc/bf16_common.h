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

// Row permutation for the A operand of a 32x32 MFMA: swapping bits 2 and 3
// of the row index makes result register i of lane l hold row
// 16*(i/8) + 8*(l/32) + i%8, so each lane's registers 8t..8t+7 cover 8
// consecutive rows: the k-slot layout of a following MFMA's operand.
__device__ inline int perm_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

constexpr float kLog2e = 1.4426950408889634f;

// ds_read_b64_tr_b16 (gfx950 LDS transpose read).  Within each group of 16
// lanes, every lane names an 8-byte segment (4 bf16); output element e of
// lane i of the group is element i%4 of the segment named by lane 4e + i/4.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ inline u32x2 ds_read_tr(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// 32x32x16 MFMA operand (lane l holds n = l%32 and k = 8*(l/32) .. +7, i.e.
// the B layout, which is also the A layout with m in place of n) read from a
// row-major LDS matrix M[k][n] with row stride `st` elements, for the block
// k0 .. k0+15, n0 .. n0+31.  Two transpose reads, rows +0..3 and +4..7.
__device__ inline u32x4 lds_operand_tr(const uint16_t* M, int st, int k0, int n0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const uint16_t* p = M + (k0 + 8 * (g >> 1) + (j >> 2)) * st + n0 + 16 * (g & 1) + 4 * (j & 3);
  const u32x2 a = ds_read_tr(p), b = ds_read_tr(p + 4 * st);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// Buffer resources: raw (stride 0) buffers whose size bounds every access in
// hardware.  Loads past `bytes` return zero and stores past it are dropped,
// so row tails need no branches.  The fourth descriptor word is the gfx9
// raw-buffer format (32-bit data format, no swizzle).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
__device__ inline u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline float bloadf(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void bstore8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
__device__ inline void bstoref(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
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
