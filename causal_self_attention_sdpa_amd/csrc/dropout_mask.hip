// The keep decisions of attention dropout written out as bytes (1 = kept),
// from the same generator code the attention kernels use (philox.h), for
// callers that inspect or replay a mask.  One thread per generator block: 8
// consecutive keys of one query.
#include "gattn_internal.h"

namespace gattn {
namespace {

__global__ __launch_bounds__(256) void dropout_mask_kernel(uint8_t* __restrict__ keep, int BH,
                                                           int T, Dropout dr) {
  const int ng = (T + 7) / 8;  // blocks per query row
  const long id = long(blockIdx.x) * 256 + threadIdx.x;
  if (id >= long(BH) * T * ng) return;
  const int g = int(id % ng);
  const long r = id / ng;  // bh * T + i
  const int i = int(r % T), bh = int(r / T);
  const uint32_t bits = keep_bits8(uint32_t(i), uint32_t(g), uint32_t(bh), dr);
  uint8_t* row = keep + r * T;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (8 * g + e < T) row[8 * g + e] = uint8_t((bits >> e) & 1u);
}

}  // namespace

hipError_t dropout_mask(uint8_t* keep, int BH, int T, const Dropout& dr, hipStream_t s) {
  const long threads = long(BH) * T * ((T + 7) / 8);
  return launch(dropout_mask_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), s, keep, BH,
                T, dr);
}

}  // namespace gattn
