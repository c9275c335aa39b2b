// Diagnostics.  mfma_loop: the achievable bf16 MFMA rate at the current clock.  Every
// wavefront runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on
// register operands (no memory traffic in the loop) and finally writes one
// float per wavefront, so the loop cannot be removed.  The benchmark reports
// this beside the published peak.
#include "gattn_internal.h"
#include "mfma16_common.h"

namespace gattn {
namespace {

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  const u32x4 a = {uint32_t(lane) * 0x00010001u, 0x3F803F80u, 0x3F003F00u, uint32_t(lane)};
  const u32x4 b = {0x3F803F80u, uint32_t(lane) << 3, 0x3E803E80u, 0x3F803F80u};
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = Bf16::mfma(a, b, acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// Diagnostic: what the vector ALU costs beside the matrix core.  Workgroups of
// 8 wavefronts, one workgroup per CU (two wavefronts per SIMD: wavefronts 0-3
// and 4-7 each span the CU's four SIMDs).  `roles` says what each half runs, on register operands only:
//   bit 0: wavefronts 0-3 run mfma_iters rounds of 4 independent bf16 MFMAs
//          (32x32x16);
//   bit 1: wavefronts 0-3 run valu_iters rounds of 16 independent vector
//          instructions of `kind` (0: v_fma_f32, 1: v_mul_f32, 2: v_exp_f32);
//   bits 2, 3: the same for wavefronts 4-7.
// A wavefront with both runs its MFMAs first.  Each wavefront writes one
// float to sink[8 * block + wavefront], so no loop can be removed.
template <int KIND>
__device__ __forceinline__ void valu_rounds(float (&x)[16], float y, float z, int iters) {
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (KIND == 0) x[i] = fmaf(x[i], y, z);
      if constexpr (KIND == 1) x[i] = x[i] * y;
      if constexpr (KIND == 2) x[i] = __builtin_amdgcn_exp2f(x[i]);
    }
    // keep the 16 chains apart (no reassociation across rounds)
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                 "+v"(x[6]), "+v"(x[7]));
    asm volatile("" : "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]),
                 "+v"(x[13]), "+v"(x[14]), "+v"(x[15]));
  }
}

__global__ __launch_bounds__(512) void issue_probe_kernel(float* __restrict__ sink, int mfma_iters,
                                                          int valu_iters, int kind, int roles,
                                                          float y, float z) {
  // 96 KB of LDS: no second workgroup fits on the CU, so each SIMD holds
  // exactly the two wavefronts named above.
  __shared__ float pin[24576];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = w < 4 ? roles & 3 : (roles >> 2) & 3;
  if (roles == 0) pin[threadIdx.x] = 0.f;  // never true (roles >= 1); keeps the array
  const u32x4 a = {uint32_t(lane) * 0x00010001u, 0x3F803F80u, 0x3F003F00u, uint32_t(lane)};
  const u32x4 b = {0x3F803F80u, uint32_t(lane) << 3, 0x3E803E80u, 0x3F803F80u};
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = float(lane) * 1e-3f + float(i) * 1e-2f;
  if (r & 1)
    for (int it = 0; it < mfma_iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Bf16::mfma(a, b, acc[i]);
    }
  if (r & 2) {
    if (kind == 0)
      valu_rounds<0>(x, y, z, valu_iters);
    else if (kind == 1)
      valu_rounds<1>(x, y, z, valu_iters);
    else
      valu_rounds<2>(x, y, z, valu_iters);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[i][e];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += x[i];
  if (roles == 0) s += pin[threadIdx.x];
  if (lane == 0) sink[blockIdx.x * 8 + w] = s;
}

}  // namespace

hipError_t mfma_loop(float* sink, int blocks, int iters, hipStream_t s) {
  return launch(mfma_loop_kernel, dim3(unsigned(blocks)), dim3(256), s, sink, iters);
}

hipError_t issue_probe(float* sink, int blocks, int mfma_iters, int valu_iters, int kind, int roles,
                       hipStream_t s) {
  return launch(issue_probe_kernel, dim3(unsigned(blocks)), dim3(512), s, sink, mfma_iters,
                valu_iters, kind, roles, 0.999f, 1e-3f);
}

}  // namespace gattn
