// float32 causal attention, forward and backward, one wavefront per row.
//
// Used for float32 tensors with any T and hs <= 128 (the tiny
// character-level shape, T = 8, hs = 8, is the intended case).  A wavefront of
// 64 lanes owns one row; lane t holds elements d = t and d = t + 64 of that
// row.  Dot products are wavefront sums (xor-butterfly shuffles), so every
// result is independent of launch order: the path is deterministic and uses
// no atomics.
//
// Tensors are addressed through Layout strides (rows of hs contiguous
// elements): q, k, v share layout li, o and dO share lo, dq, dk, dv share lg;
// lse, D and L2 are contiguous (B, H, T).
//
// Per row i (query) or column j (key) of one (b, h) slice:
//   forward  : online softmax over keys j <= i (tril mask, "Let's build GPT"
//              summary page 48:54 / 55:20; softmax rows 51:04), scores scaled
//              by `scale` (1:17:18), values summed with the weights (1:10:15).
//   backward : chain rule; P is recomputed as exp(s - lse).
// Dropout (dr.thr != 0, philox.h): weight (i, j) is kept by its own
// generator decision and kept weights are multiplied by dr.zs in the value
// sum; the backward uses dV = (P*Z)^T dO, dS = P * (Z * dO V^T - D).
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

// One wavefront per query row.  Tq queries against Tk >= Tq keys: query i
// is the token at position Tk - Tq + i and sees keys j <= Tk - Tq + i
// (Tq = Tk: the causal forward).
template <int NPL>
__global__ __launch_bounds__(64 * kWaves) void f32_fwd_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int BH, int H, int Tq, int Tk, int hs,
    float scale, Layout lq, Layout lk, Layout lo, Dropout dr) {
  const int lane = threadIdx.x & 63;
  const long row = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= long(BH) * Tq) return;  // uniform per wavefront
  const int bh = int(row / Tq);
  const int i = int(row - long(bh) * Tq);
  const int64_t sk = slice_offset(lk, bh, H);
  const float* kb = k + sk;
  const float* vb = v + sk;
  float qr[NPL], acc[NPL];
  load_row<NPL>(q + slice_offset(lq, bh, H) + i * lq.st, hs, lane, qr);
#pragma unroll
  for (int e = 0; e < NPL; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int last = Tk - Tq + i;
  for (int j = 0; j <= last; ++j) {
    const float s = wave_sum(row_dot<NPL>(qr, kb + j * lk.st, hs, lane)) * scale;
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn);  // m = -inf on the first key: alpha = 0
    const float p = expf(s - mn);
    l = l * alpha + p;
    const float pk = dr.thr == 0 || keep_one(uint32_t(last), uint32_t(j), uint32_t(bh), dr) ? p
                                                                                             : 0.f;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      float vv = d < hs ? vb[j * lk.st + d] : 0.f;
      acc[e] = fmaf(pk, vv, acc[e] * alpha);
    }
    m = mn;
  }
  const float inv = (dr.thr == 0 ? 1.f : dr.zs) / l;
  float* orow = o + slice_offset(lo, bh, H) + i * lo.st;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < hs) orow[d] = acc[e] * inv;
  }
  if (lse != nullptr && lane == 0) lse[row] = m + logf(l);
}

// D[i] = <dO_i, o_i> and L2[i] = lse[i] * log2(e), one wavefront per row.
template <int NPL>
__global__ __launch_bounds__(64 * kWaves) void f32_pre_kernel(
    const float* __restrict__ o, const float* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ D, float* __restrict__ L2, int BH, int H, int T, int hs, Layout lo) {
  const int lane = threadIdx.x & 63;
  const long row = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= long(BH) * T) return;
  const int bh = int(row / T);
  const int i = int(row - long(bh) * T);
  const int64_t off = slice_offset(lo, bh, H) + i * lo.st;
  float a[NPL];
  load_row<NPL>(dO + off, hs, lane, a);
  const float s = wave_sum(row_dot<NPL>(a, o + off, hs, lane));
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
    float* __restrict__ dk, float* __restrict__ dv, int BH, int H, int T, int hs, float scale,
    Layout li, Layout lo, Layout lg, Dropout dr) {
  const float c = scale * 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const long row = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= long(BH) * T) return;
  const int bh = int(row / T);
  const int j = int(row - long(bh) * T);
  const int64_t si = slice_offset(li, bh, H);
  const float* qb = q + si;
  const float* ob = dO + slice_offset(lo, bh, H);
  const long rb = long(bh) * T;  // row base of the (B, H, T) vectors
  float kr[NPL], vr[NPL], ak[NPL], av[NPL];
  load_row<NPL>(k + si + j * li.st, hs, lane, kr);
  load_row<NPL>(v + si + j * li.st, hs, lane, vr);
#pragma unroll
  for (int e = 0; e < NPL; ++e) ak[e] = av[e] = 0.f;
  for (int i = j; i < T; ++i) {
    float s = row_dot<NPL>(kr, qb + i * li.st, hs, lane);
    float dp = row_dot<NPL>(vr, ob + i * lo.st, hs, lane);
    wave_sum2(s, dp);
    const float p = exp2f(fmaf(s, c, -L2[rb + i]));
    const bool kept = dr.thr == 0 || keep_one(uint32_t(i), uint32_t(j), uint32_t(bh), dr);
    const float pk = kept ? p : 0.f;
    const float ds = p * ((kept ? dp * (dr.thr == 0 ? 1.f : dr.zs) : 0.f) - D[rb + i]);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      float qq = d < hs ? qb[i * li.st + d] : 0.f;
      float gg = d < hs ? ob[i * lo.st + d] : 0.f;
      av[e] = fmaf(pk, gg, av[e]);
      ak[e] = fmaf(ds, qq, ak[e]);
    }
  }
  const float zv = dr.thr == 0 ? 1.f : dr.zs;
  const int64_t go = slice_offset(lg, bh, H) + j * lg.st;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < hs) {
      dk[go + d] = ak[e] * scale;
      dv[go + d] = av[e] * zv;
    }
  }
}

// dQ_i: one wavefront per query row i, loop over keys j <= i.
template <int NPL>
__global__ __launch_bounds__(64 * kWaves) void f32_dq_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ D,
    float* __restrict__ dq, int BH, int H, int T, int hs, float scale, Layout li, Layout lo,
    Layout lg, Dropout dr) {
  const int lane = threadIdx.x & 63;
  const long row = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= long(BH) * T) return;
  const int bh = int(row / T);
  const int i = int(row - long(bh) * T);
  const int64_t si = slice_offset(li, bh, H);
  const float* kb = k + si;
  const float* vb = v + si;
  float qr[NPL], gr[NPL], aq[NPL];
  load_row<NPL>(q + si + i * li.st, hs, lane, qr);
  load_row<NPL>(dO + slice_offset(lo, bh, H) + i * lo.st, hs, lane, gr);
#pragma unroll
  for (int e = 0; e < NPL; ++e) aq[e] = 0.f;
  const float li_ = lse[row], Di = D[row];
  for (int j = 0; j <= i; ++j) {
    float s = row_dot<NPL>(qr, kb + j * li.st, hs, lane);
    float dp = row_dot<NPL>(gr, vb + j * li.st, hs, lane);
    wave_sum2(s, dp);
    const float p = expf(s * scale - li_);
    const bool kept = dr.thr == 0 || keep_one(uint32_t(i), uint32_t(j), uint32_t(bh), dr);
    const float ds = p * ((kept ? dp * (dr.thr == 0 ? 1.f : dr.zs) : 0.f) - Di);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      float kk = d < hs ? kb[j * li.st + d] : 0.f;
      aq[e] = fmaf(ds, kk, aq[e]);
    }
  }
  float* qrow = dq + slice_offset(lg, bh, H) + i * lg.st;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < hs) qrow[d] = aq[e] * scale;
  }
}

dim3 rows_grid(int BH, int T) {
  long rows = long(BH) * T;
  return dim3(unsigned((rows + kWaves - 1) / kWaves));
}

}  // namespace

hipError_t f32_fwd(const float* q, const float* k, const float* v, float* o, float* lse, int BH,
                   int H, int Tq, int Tk, int hs, float scale, Layout lq, Layout lk, Layout lo,
                   const Dropout& dr, hipStream_t s) {
  auto kern = hs <= 64 ? f32_fwd_kernel<1> : f32_fwd_kernel<2>;
  return launch(kern, rows_grid(BH, Tq), dim3(64 * kWaves), s, q, k, v, o, lse, BH, H, Tq, Tk, hs,
                scale, lq, lk, lo, dr);
}

hipError_t f32_bwd_pre(const float* o, const float* dO, const float* lse, float* D, float* L2,
                       int BH, int H, int T, int hs, Layout lo, hipStream_t s) {
  if (hs <= 64)
    return launch(f32_pre_kernel<1>, rows_grid(BH, T), dim3(64 * kWaves), s, o, dO, lse, D, L2, BH,
                  H, T, hs, lo);
  return launch(f32_pre_kernel<2>, rows_grid(BH, T), dim3(64 * kWaves), s, o, dO, lse, D, L2, BH, H,
                T, hs, lo);
}

hipError_t f32_bwd_dkdv(const float* q, const float* k, const float* v, const float* dO,
                        const float* D, const float* L2, float* dk, float* dv, int BH, int H,
                        int T, int hs, float scale, Layout li, Layout lo, Layout lg,
                        const Dropout& dr, hipStream_t s) {
  if (hs <= 64)
    return launch(f32_dkdv_kernel<1>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, dO, D, L2,
                  dk, dv, BH, H, T, hs, scale, li, lo, lg, dr);
  return launch(f32_dkdv_kernel<2>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, dO, D, L2, dk,
                dv, BH, H, T, hs, scale, li, lo, lg, dr);
}

hipError_t f32_bwd_dq(const float* q, const float* k, const float* v, const float* dO,
                      const float* lse, const float* D, float* dq, int BH, int H, int T, int hs,
                      float scale, Layout li, Layout lo, Layout lg, const Dropout& dr,
                      hipStream_t s) {
  if (hs <= 64)
    return launch(f32_dq_kernel<1>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, dO, lse, D,
                  dq, BH, H, T, hs, scale, li, lo, lg, dr);
  return launch(f32_dq_kernel<2>, rows_grid(BH, T), dim3(64 * kWaves), s, q, k, v, dO, lse, D, dq,
                BH, H, T, hs, scale, li, lo, lg, dr);
}

}  // namespace gattn
