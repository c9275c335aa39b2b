// bf16 backward helper kernels, both bound by HBM bandwidth:
//   preprocess: D[i] = sum_d dO[i][d] * O[i][d] in f32 (the row term of the
//               softmax backward, dS = P (dP - D)), and the f32 dQ
//               accumulator rows set to zero (a fill kernel rather than a
//               memset node, so the call is safe to capture in a graph);
//   finalize  : dQ accumulator (f32) -> dq (bf16, round to nearest even).
// Each thread moves 16-byte vectors; consecutive threads touch consecutive
// addresses.
#include "bf16_common.h"
#include "gattn_internal.h"

namespace gattn {
namespace {

constexpr int kThreads = 256;

// HS/8 threads per row, each owns 8 consecutive elements (one 16-byte load).
template <int HS>
__global__ __launch_bounds__(kThreads) void bf16_pre_kernel(const uint16_t* __restrict__ o,
                                                           const uint16_t* __restrict__ dO,
                                                           float* __restrict__ D,
                                                           float* __restrict__ dq_acc,
                                                           long rows) {
  constexpr int TPR = HS / 8;  // threads per row (power of two)
  const long gid = long(blockIdx.x) * kThreads + threadIdx.x;
  const long row = gid / TPR;
  const int part = int(gid % TPR);
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * HS + part * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * HS + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s = fmaf(bf16lo(a[w]), bf16lo(b[w]), s);
      s = fmaf(bf16hi(a[w]), bf16hi(b[w]), s);
    }
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4* dst = reinterpret_cast<f32x4*>(dq_acc + row * HS + part * 8);
    dst[0] = z;
    dst[1] = z;
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (row < rows && part == 0) D[row] = s;
}

__global__ __launch_bounds__(kThreads) void bf16_fin_kernel(const float* __restrict__ acc,
                                                           uint16_t* __restrict__ dq, long n8) {
  const long i = long(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n8) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(acc) + 2 * i;
  const f32x4 a = src[0], b = src[1];
  u32x4 r = {pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]),
             pack_bf16(b[2], b[3])};
  reinterpret_cast<u32x4*>(dq)[i] = r;
}

}  // namespace

hipError_t bf16_bwd_pre(const uint16_t* o, const uint16_t* dO, float* D, float* dq_acc, int BH,
                        int T, int hs, hipStream_t s) {
  const long rows = long(BH) * T;
  const long threads = rows * (hs / 8);
  const dim3 grid(unsigned((threads + kThreads - 1) / kThreads));
  if (hs == 64) return launch(bf16_pre_kernel<64>, grid, dim3(kThreads), s, o, dO, D, dq_acc, rows);
  return launch(bf16_pre_kernel<32>, grid, dim3(kThreads), s, o, dO, D, dq_acc, rows);
}

hipError_t bf16_bwd_fin(const float* dq_acc, uint16_t* dq, int BH, int T, int hs, hipStream_t s) {
  const long n8 = long(BH) * T * hs / 8;
  return launch(bf16_fin_kernel, dim3(unsigned((n8 + kThreads - 1) / kThreads)), dim3(kThreads), s,
                dq_acc, dq, n8);
}

}  // namespace gattn
