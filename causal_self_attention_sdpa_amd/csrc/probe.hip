// Diagnostic: the achievable bf16 MFMA rate at the current clock.  Every
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

}  // namespace

hipError_t mfma_loop(float* sink, int blocks, int iters, hipStream_t s) {
  return launch(mfma_loop_kernel, dim3(unsigned(blocks)), dim3(256), s, sink, iters);
}

}  // namespace gattn
