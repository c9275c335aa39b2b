// Internal declarations shared by the gattn kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <tuple>

namespace gattn {

// Launch a __global__ function through hipLaunchKernel so that the launch
// status comes back directly (no reliance on the thread's sticky last error).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
  void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply(
      [&](auto&... x) {
        int n = 0;
        ((argv[n++] = static_cast<void*>(&x)), ...);
      },
      vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, 0, stream);
}

// Backward workspace: [D = rowsum(dO * O)][L2 = lse * log2(e)], each float32
// (B, H, T) and starting on a 256-byte boundary.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t ws_part_bytes(int B, int H, int T) {
  return align256(sizeof(float) * size_t(B) * H * T);
}

// ---- float32 path (any hs <= 128, any T; wave per row; deterministic) ----
hipError_t f32_fwd(const float* q, const float* k, const float* v, float* o, float* lse, int BH,
                   int T, int hs, float scale, hipStream_t s);
hipError_t f32_bwd_pre(const float* o, const float* dO, const float* lse, float* D, float* L2,
                       int BH, int T, int hs, hipStream_t s);
hipError_t f32_bwd_dkdv(const float* q, const float* k, const float* v, const float* dO,
                        const float* D, const float* L2, float* dk, float* dv, int BH, int T,
                        int hs, float scale, hipStream_t s);
hipError_t f32_bwd_dq(const float* q, const float* k, const float* v, const float* dO,
                      const float* lse, const float* D, float* dq, int BH, int T, int hs,
                      float scale, hipStream_t s);

// ---- bf16 path (hs in {32, 64}; MFMA) ----
hipError_t bf16_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                    float* lse, int BH, int T, int hs, float scale, hipStream_t s);
hipError_t bf16_bwd_pre(const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                        float* L2, int BH, int T, int hs, hipStream_t s);
hipError_t bf16_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, const float* D, const float* L2, uint16_t* dk,
                         uint16_t* dv, int BH, int T, int hs, float scale, hipStream_t s);
hipError_t bf16_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                       float* L2, uint16_t* dq, int BH, int T, int hs, float scale,
                       hipStream_t s);

}  // namespace gattn
