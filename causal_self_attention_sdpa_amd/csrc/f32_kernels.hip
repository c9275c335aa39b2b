// float32 causal attention, forward and backward, one wavefront per row.
//
// Used for float32 tensors with any T and hs <= 128 (the tiny
// character-level shape, T = 8, hs = 8, is the intended case).  A wavefront of
// 64 lanes owns one row; lane t holds elements d = t and d = t + 64 of that
// row.  Dot products are wavefront sums (xor-butterfly shuffles), so every
// result is independent of launch order: the path is deterministic and uses
// no atomics.
//
// Per row i (query) or column j (key) of one (b, h) slice:
//   forward  : online softmax over keys j <= i (tril mask, "Let's build GPT"
//              summary page 48:54 / 55:20; softmax rows 51:04), scores scaled
//              by `scale` (1:17:18), values summed with the weights (1:10:15).
//   backward : chain rule; P is recomputed as exp(s - lse).
#include "gattn_internal.h"

#include <cmath>

namespace gattn {
namespace {

constexpr int kWaves = 4;  // wavefronts per workgroup

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ inline void wave_sum2(float& a, float& b) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
  }
}

template <int NPL>
__device__ inline void load_row(const float* __restrict__ p, int hs, int lane, float (&r)[NPL]) {
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    r[e] = d < hs ? p[d] : 0.f;
  }
}

template <int NPL>
__device__ inline float row_dot(const float (&a)[NPL], const float* __restrict__ p, int hs,
                                int lane) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < hs) s = fmaf(a[e], p[d], s);
  }
  return s;
}

// One wavefront per query row.
template <int NPL>
__global__ __launch_bounds__(64 * kWaves) void f32_fwd_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int BH, int T, int hs, float scale) {
  const int lane = threadIdx.x & 63;
  const long row = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= long(BH) * T) return;  // uniform per wavefront
  const long bh = row / T;
  const int i = int(row - bh * T);
  const float* kb = k + bh * T * hs;
  const float* vb = v + bh * T * hs;
  float qr[NPL], acc[NPL];
  load_row<NPL>(q + row * hs, hs, lane, qr);
#pragma unroll
  for (int e = 0; e < NPL; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= i; ++j) {
    const float s = wave_sum(row_dot<NPL>(qr, kb + long(j) * hs, hs, lane)) * scale;
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn);  // m = -inf on the first key: alpha = 0
    const float p = expf(s - mn);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      float vv = d < hs ? vb[long(j) * hs + d] : 0.f;
      acc[e] = fmaf(p, vv, acc[e] * alpha);
    }
    m = mn;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < hs) o[row * hs + d] = acc[e] * inv;
  }
  if (lse != nullptr && lane == 0) lse[row] = m + logf(l);
}

// D[i] = <dO_i, o_i> and L2[i] = lse[i] * log2(e), one wavefront per row.
template <int NPL>
__global__ __launch_bounds__(64 * kWaves) void f32_pre_kernel(
    const float* __restrict__ o, const float* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ D, float* __restrict__ L2, int BH, int T, int hs) {
  const int lane = threadIdx.x & 63;
  const long row = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= long(BH) * T) return;
  float a[NPL];
  load_row<NPL>(dO + row * hs, hs, lane, a);
  const float s = wave_sum(row_dot<NPL>(a, o + row * hs, hs, lane));
  if (lane == 0) {
    D[row] = s;
    L2[row] = lse[row] * 1.4426950408889634f;
  }
}

// dK_j, dV_j: one wavefront per key row j, loop over queries i >= j.
// P = exp2(s * scale * log2(e) - L2) with L2 = lse * log2(e) from the workspace.
template <int NPL>
__global__ __launch_bounds__(64 * kWaves) void f32_dkdv_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ D, const float* __restrict__ L2,
    float* __restrict__ dk, float* __restrict__ dv, int BH, int T, int hs, float scale) {
  const float c = scale * 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const long row = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= long(BH) * T) return;
  const long bh = row / T;
  const int j = int(row - bh * T);
  const float* qb = q + bh * T * hs;
  const float* ob = dO + bh * T * hs;
  float kr[NPL], vr[NPL], ak[NPL], av[NPL];
  load_row<NPL>(k + row * hs, hs, lane, kr);
  load_row<NPL>(v + row * hs, hs, lane, vr);
#pragma unroll
  for (int e = 0; e < NPL; ++e) ak[e] = av[e] = 0.f;
  for (int i = j; i < T; ++i) {
    float s = row_dot<NPL>(kr, qb + long(i) * hs, hs, lane);
    float dp = row_dot<NPL>(vr, ob + long(i) * hs, hs, lane);
    wave_sum2(s, dp);
    const float p = exp2f(fmaf(s, c, -L2[bh * T + i]));
    const float ds = p * (dp - D[bh * T + i]);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      float qq = d < hs ? qb[long(i) * hs + d] : 0.f;
      float gg = d < hs ? ob[long(i) * hs + d] : 0.f;
      av[e] = fmaf(p, gg, av[e]);
      ak[e] = fmaf(ds, qq, ak[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < hs) {
      dk[row * hs + d] = ak[e] * scale;
      dv[row * hs + d] = av[e];
    }
  }
}

// dQ_i: one wavefront per query row i, loop over keys j <= i.
template <int NPL>
__global__ __launch_bounds__(64 * kWaves) void f32_dq_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ D,
    float* __restrict__ dq, int BH, int T, int hs, float scale) {
  const int lane = threadIdx.x & 63;
  const long row = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= long(BH) * T) return;
  const long bh = row / T;
  const int i = int(row - bh * T);
  const float* kb = k + bh * T * hs;
  const float* vb = v + bh * T * hs;
  float qr[NPL], gr[NPL], aq[NPL];
  load_row<NPL>(q + row * hs, hs, lane, qr);
  load_row<NPL>(dO + row * hs, hs, lane, gr);
#pragma unroll
  for (int e = 0; e < NPL; ++e) aq[e] = 0.f;
  const float li = lse[row], Di = D[row];
  for (int j = 0; j <= i; ++j) {
    float s = row_dot<NPL>(qr, kb + long(j) * hs, hs, lane);
    float dp = row_dot<NPL>(gr, vb + long(j) * hs, hs, lane);
    wave_sum2(s, dp);
    const float p = expf(s * scale - li);
    const float ds = p * (dp - Di);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      float kk = d < hs ? kb[long(j) * hs + d] : 0.f;
      aq[e] = fmaf(ds, kk, aq[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < hs) dq[row * hs + d] = aq[e] * scale;
  }
}

dim3 rows_grid(int BH, int T) {
  long rows = long(BH) * T;
  return dim3(unsigned((rows + kWaves - 1) / kWaves));
}

}  // namespace

hipError_t f32_fwd(const float* q, const float* k, const float* v, float* o, float* lse, int BH,
                   int T, int hs, float scale, hipStream_t s) {
  if (hs <= 64)
    return launch(f32_fwd_kernel<1>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, o, lse, BH,
                  T, hs, scale);
  return launch(f32_fwd_kernel<2>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, o, lse, BH, T,
                hs, scale);
}

hipError_t f32_bwd_pre(const float* o, const float* dO, const float* lse, float* D, float* L2,
                       int BH, int T, int hs, hipStream_t s) {
  if (hs <= 64)
    return launch(f32_pre_kernel<1>, rows_grid(BH, T), dim3(64 * kWaves), s, o, dO, lse, D, L2, BH,
                  T, hs);
  return launch(f32_pre_kernel<2>, rows_grid(BH, T), dim3(64 * kWaves), s, o, dO, lse, D, L2, BH, T,
                hs);
}

hipError_t f32_bwd_dkdv(const float* q, const float* k, const float* v, const float* dO,
                        const float* D, const float* L2, float* dk, float* dv, int BH, int T,
                        int hs, float scale, hipStream_t s) {
  if (hs <= 64)
    return launch(f32_dkdv_kernel<1>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, dO, D, L2,
                  dk, dv, BH, T, hs, scale);
  return launch(f32_dkdv_kernel<2>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, dO, D, L2, dk,
                dv, BH, T, hs, scale);
}

hipError_t f32_bwd_dq(const float* q, const float* k, const float* v, const float* dO,
                      const float* lse, const float* D, float* dq, int BH, int T, int hs,
                      float scale, hipStream_t s) {
  if (hs <= 64)
    return launch(f32_dq_kernel<1>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, dO, lse, D,
                  dq, BH, T, hs, scale);
  return launch(f32_dq_kernel<2>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, dO, lse, D, dq,
                BH, T, hs, scale);
}

}  // namespace gattn
