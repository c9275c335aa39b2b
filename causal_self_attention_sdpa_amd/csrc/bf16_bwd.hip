// bf16 causal attention backward on gfx950 MFMA: three kernels, no atomics.
//
// The pages state only that the model is trained with a backward pass; the
// gradients are the chain rule of the forward ("Let's build GPT" summary
// page: tril mask 48:54 / 55:20, row softmax 51:04, scaled q.k 1:06:16 /
// 1:17:18, weighted values 1:10:15):
//   P  = exp(scale * Q K^T - lse)    recomputed from the forward's lse,
//                                    exactly 0 above the diagonal
//   D  = rowsum(dO * O)              (preprocess kernel)
//   dP = dO V^T,   dS = P * (dP - D)
//   dV = P^T dO,   dK = scale * dS^T Q        (dK/dV kernel, per key tile)
//   dQ = scale * dS K                          (dQ kernel, per query tile)
// Splitting dQ from dK/dV costs a second recomputation of S and dP, and in
// exchange removes float32 atomics (which on this chip are executed past the
// per-XCD L2s), the zeroing and conversion passes of an accumulator, and the
// LDS round trip of dS; every output is deterministic.
//
// Both main kernels stream tiles through double-buffered LDS with one barrier
// per step: the loads for step t+1 are in flight (in registers) while step t
// computes.  Global accesses go through buffer resources sized to one (b, h)
// slice, so rows past T read as zero and their stores are dropped.
#include <cmath>

#include "bf16_common.h"
#include "gattn_internal.h"

namespace gattn {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// D[i] = sum_d dO[i][d] * O[i][d]; HS/8 threads per row, 16-byte loads.
template <int HS>
__global__ __launch_bounds__(kThreads) void bf16_pre_kernel(const uint16_t* __restrict__ o,
                                                           const uint16_t* __restrict__ dO,
                                                           float* __restrict__ D, long rows) {
  constexpr int TPR = HS / 8;
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
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (row < rows && part == 0) D[row] = s;
}

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup = 4 wavefronts = 128 keys of one (b, h); wavefront w
// keeps keys k0 + 32w .. +31 (K, V as MFMA B operands) and their dK^T, dV^T
// accumulators in registers.  Steps walk 64-query tiles from the diagonal to
// T.  Per step and 32-query block:
//   S = Q K^T, dP = dO V^T          C[query][key]; Q, dO rows read from LDS in
//                                   perm_row order, so each lane's registers
//                                   8t..8t+7 are 8 consecutive queries
//   P, dS (f32, registers) -> bf16  exactly the B operand of the next MFMAs
//   dV^T += dO^T P, dK^T += Q^T dS  C[d][key]; dO^T, Q^T via LDS transpose reads
template <int HS>
struct DkdvCfg {
  static constexpr int NW = 4;
  static constexpr int BN = 32 * NW;              // keys per workgroup
  static constexpr int BQ = 64;                   // queries per step
  static constexpr int QB = BQ / 32;
  static constexpr int KSTEP = HS / 16;
  static constexpr int DB = HS / 32;
  static constexpr int ST = HS + 8;               // LDS row stride (elements)
  static constexpr int LPT = BQ * HS / 8 / kThreads;  // 16-byte chunks per thread per tensor
  static_assert(LPT >= 1, "tile shape");
};

template <int HS, bool MASK>
__device__ inline void dkdv_block(const uint16_t* Qb, const uint16_t* Gb, const float* Lb,
                                  const float* Db, int qb, int qs0, int krow, int prow, int lane,
                                  int h, float c, const u32x4 (&kf)[HS / 16],
                                  const u32x4 (&vf)[HS / 16], f32x16 (&dka)[HS / 32],
                                  f32x16 (&dva)[HS / 32]) {
  using C = DkdvCfg<HS>;
  const f32x16 zero = {};
  f32x16 s = zero, dp = zero;
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks) {
    const int off = (qb * 32 + prow) * C::ST + 16 * ks + 8 * h;
    s = mfma32(*reinterpret_cast<const u32x4*>(Qb + off), kf[ks], s);
    dp = mfma32(*reinterpret_cast<const u32x4*>(Gb + off), vf[ks], dp);
  }
  u32x4 pp[2], dsp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int ql = qb * 32 + 16 * t + 8 * h;  // local index of this lane's run of 8 queries
    const f32x4 l0 = *reinterpret_cast<const f32x4*>(Lb + ql);
    const f32x4 l1 = *reinterpret_cast<const f32x4*>(Lb + ql + 4);
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(Db + ql);
    const f32x4 d1 = *reinterpret_cast<const f32x4*>(Db + ql + 4);
    float pv[8], dsv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float le = e < 4 ? l0[e] : l1[e - 4];
      const float De = e < 4 ? d0[e] : d1[e - 4];
      float p = __builtin_amdgcn_exp2f(fmaf(s[8 * t + e], c, -le));
      if (MASK && krow > qs0 + ql + e) p = 0.f;
      pv[e] = p;
      dsv[e] = p * (dp[8 * t + e] - De);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pp[t][e] = pack_bf16(pv[2 * e], pv[2 * e + 1]);
      dsp[t][e] = pack_bf16(dsv[2 * e], dsv[2 * e + 1]);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int k0 = qb * 32 + 16 * t;
      dva[db] = mfma32(lds_operand_tr(Gb, C::ST, k0, db * 32, lane), pp[t], dva[db]);
      dka[db] = mfma32(lds_operand_tr(Qb, C::ST, k0, db * 32, lane), dsp[t], dka[db]);
    }
}

template <int HS>
__global__ __launch_bounds__(kThreads, 2) void bf16_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Dg, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int BH, int T, float scale) {
  using C = DkdvCfg<HS>;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][C::BQ * C::ST];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[2][C::BQ * C::ST];
  __shared__ __attribute__((aligned(16))) float Ls[2][C::BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][C::BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  // Key tiles near the start have the most query tiles below the diagonal.
  const int kt = int(blockIdx.x) / BH;
  const int bh = int(blockIdx.x) % BH;
  const long base = long(bh) * T * HS;
  const uint32_t slice_bytes = uint32_t(T) * HS * 2;
  const rsrc_t rq = make_rsrc(q + base, slice_bytes), rk = make_rsrc(k + base, slice_bytes);
  const rsrc_t rv = make_rsrc(v + base, slice_bytes), rg = make_rsrc(dO + base, slice_bytes);
  const rsrc_t rl = make_rsrc(lse + long(bh) * T, uint32_t(T) * 4);
  const rsrc_t rd = make_rsrc(Dg + long(bh) * T, uint32_t(T) * 4);

  const int k0 = kt * C::BN;
  const int kw0 = k0 + 32 * w;
  const int krow = kw0 + n;
  const float c = scale * kLog2e;

  u32x4 kf[C::KSTEP], vf[C::KSTEP];
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks) {
    const uint32_t off = uint32_t(krow * HS + 16 * ks + 8 * h) * 2;
    kf[ks] = bload16(rk, off);
    vf[ks] = bload16(rv, off);
  }
  f32x16 dka[C::DB], dva[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dka[db] = dva[db] = f32x16{};

  u32x4 qr[C::LPT], gr[C::LPT];
  float lr = 0.f, dr = 0.f;
  auto gload = [&](int qt) {
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const int ch = tid + kThreads * j, row = ch / (HS / 8), col = ch % (HS / 8);
      const uint32_t off = uint32_t((qt * C::BQ + row) * HS + col * 8) * 2;
      qr[j] = bload16(rq, off);
      gr[j] = bload16(rg, off);
    }
    if (tid < C::BQ) {
      const int qi = qt * C::BQ + tid;
      const float l = bloadf(rl, uint32_t(qi) * 4);
      lr = qi < T ? l * kLog2e : INFINITY;  // rows past T: P = exp2(-inf) = 0
      dr = bloadf(rd, uint32_t(qi) * 4);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const int ch = tid + kThreads * j, row = ch / (HS / 8), col = ch % (HS / 8);
      *reinterpret_cast<u32x4*>(&Qs[buf][row * C::ST + col * 8]) = qr[j];
      *reinterpret_cast<u32x4*>(&Gs[buf][row * C::ST + col * 8]) = gr[j];
    }
    if (tid < C::BQ) {
      Ls[buf][tid] = lr;
      Ds[buf][tid] = dr;
    }
  };

  const int nqt = (T + C::BQ - 1) / C::BQ;
  const int qt0 = k0 / C::BQ;
  const int prow = perm_row(n);
  gload(qt0);
  lstore(0);
  __syncthreads();
  for (int qt = qt0; qt < nqt; ++qt) {
    const int buf = (qt - qt0) & 1;
    if (qt + 1 < nqt) gload(qt + 1);
    const int qs0 = qt * C::BQ;
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const int qbase = qs0 + qb * 32;
      if (kw0 > qbase + 31) continue;  // all of this wavefront's keys lie after the block
      if (kw0 + 31 > qbase)
        dkdv_block<HS, true>(Qs[buf], Gs[buf], Ls[buf], Ds[buf], qb, qs0, krow, prow, lane, h,
                             c, kf, vf, dka, dva);
      else
        dkdv_block<HS, false>(Qs[buf], Gs[buf], Ls[buf], Ds[buf], qb, qs0, krow, prow, lane, h,
                              c, kf, vf, dka, dva);
    }
    if (qt + 1 < nqt) lstore(buf ^ 1);
    __syncthreads();
  }

  // dK^T / dV^T register i of lane (n, h): column d = db*32 + 8*(i/4) + 4h + i%4, key krow.
  const rsrc_t wk = make_rsrc(dk + base, slice_bytes), wv = make_rsrc(dv + base, slice_bytes);
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = uint32_t(krow * HS + db * 32 + 8 * g + 4 * h) * 2;
      bstore8(wv, off, u32x2{pack_bf16(dva[db][4 * g], dva[db][4 * g + 1]),
                             pack_bf16(dva[db][4 * g + 2], dva[db][4 * g + 3])});
      bstore8(wk, off, u32x2{pack_bf16(dka[db][4 * g] * scale, dka[db][4 * g + 1] * scale),
                             pack_bf16(dka[db][4 * g + 2] * scale, dka[db][4 * g + 3] * scale)});
    }
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 4 wavefronts = 128 queries of one (b, h); wavefront w keeps
// queries r0 + 32w .. +31 (Q^T and dO^T as MFMA B operands, lse and D as
// per-lane scalars) and the dQ^T accumulator in registers.  Steps walk
// 64-key tiles from 0 to the diagonal.  Per step and 32-key block:
//   S^T = K Q^T, dP^T = V dO^T      C[key][query]; K, V rows from LDS in
//                                   perm_row order (8 consecutive keys per
//                                   lane in registers 8t..8t+7)
//   dS^T (f32) -> bf16               the B operand of
//   dQ^T += K^T dS^T                 C[d][query]; K^T via LDS transpose reads
template <int HS>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int BM = 32 * NW;              // queries per workgroup
  static constexpr int BN = 64;                   // keys per step
  static constexpr int KSTEP = HS / 16;
  static constexpr int DB = HS / 32;
  static constexpr int ST = HS + 8;
  static constexpr int KPT = BN * HS / 8 / kThreads;
  static_assert(KPT >= 1, "tile shape");
};

template <int HS, bool MASK>
__device__ inline void dq_step(const uint16_t* Kb, const uint16_t* Vb, int key0, int qrow,
                               int prow, int lane, int h, float c, float lse2, float Dq,
                               const u32x4 (&qf)[HS / 16], const u32x4 (&gf)[HS / 16],
                               f32x16 (&dqa)[HS / 32]) {
  using C = DqCfg<HS>;
  const f32x16 zero = {};
  u32x4 dsp[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 st = zero, dpt = zero;
#pragma unroll
    for (int ks = 0; ks < C::KSTEP; ++ks) {
      const int off = (kb * 32 + prow) * C::ST + 16 * ks + 8 * h;
      st = mfma32(*reinterpret_cast<const u32x4*>(Kb + off), qf[ks], st);
      dpt = mfma32(*reinterpret_cast<const u32x4*>(Vb + off), gf[ks], dpt);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float p = __builtin_amdgcn_exp2f(fmaf(st[8 * t + e], c, -lse2));
        if (MASK && key0 + kb * 32 + 16 * t + 8 * h + e > qrow) p = 0.f;
        dsv[e] = p * (dpt[8 * t + e] - Dq);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dsp[kb][t][e] = pack_bf16(dsv[2 * e], dsv[2 * e + 1]);
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        dqa[db] = mfma32(lds_operand_tr(Kb, C::ST, kb * 32 + 16 * t, db * 32, lane), dsp[kb][t],
                         dqa[db]);
}

template <int HS>
__global__ __launch_bounds__(kThreads, 2) void bf16_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Dg, uint16_t* __restrict__ dq,
    int BH, int T, float scale) {
  using C = DqCfg<HS>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::BN * C::ST];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][C::BN * C::ST];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int nqt = (T + C::BM - 1) / C::BM;
  const int qt = nqt - 1 - int(blockIdx.x) / BH;  // heaviest query tiles first
  const int bh = int(blockIdx.x) % BH;
  const long base = long(bh) * T * HS;
  const uint32_t slice_bytes = uint32_t(T) * HS * 2;
  const rsrc_t rq = make_rsrc(q + base, slice_bytes), rk = make_rsrc(k + base, slice_bytes);
  const rsrc_t rv = make_rsrc(v + base, slice_bytes), rg = make_rsrc(dO + base, slice_bytes);

  const int r0 = qt * C::BM;
  const int q0 = r0 + 32 * w;
  const int qrow = q0 + n;
  const float c = scale * kLog2e;
  u32x4 qf[C::KSTEP], gf[C::KSTEP];
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks) {
    const uint32_t off = uint32_t(qrow * HS + 16 * ks + 8 * h) * 2;
    qf[ks] = bload16(rq, off);
    gf[ks] = bload16(rg, off);
  }
  const float lraw = bloadf(make_rsrc(lse + long(bh) * T, uint32_t(T) * 4), uint32_t(qrow) * 4);
  const float lse2 = qrow < T ? lraw * kLog2e : INFINITY;
  const float Dq = bloadf(make_rsrc(Dg + long(bh) * T, uint32_t(T) * 4), uint32_t(qrow) * 4);
  f32x16 dqa[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dqa[db] = f32x16{};

  u32x4 kr[C::KPT], vr[C::KPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < C::KPT; ++j) {
      const int ch = tid + kThreads * j, row = ch / (HS / 8), col = ch % (HS / 8);
      const uint32_t off = uint32_t((kt * C::BN + row) * HS + col * 8) * 2;
      kr[j] = bload16(rk, off);
      vr[j] = bload16(rv, off);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < C::KPT; ++j) {
      const int ch = tid + kThreads * j, row = ch / (HS / 8), col = ch % (HS / 8);
      *reinterpret_cast<u32x4*>(&Ks[buf][row * C::ST + col * 8]) = kr[j];
      *reinterpret_cast<u32x4*>(&Vs[buf][row * C::ST + col * 8]) = vr[j];
    }
  };

  const int nkt = (min(r0 + C::BM, T) - 1) / C::BN + 1;
  const int prow = perm_row(n);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const int key0 = kt * C::BN;
    if (q0 < T && key0 <= q0 + 31) {
      if (key0 + C::BN - 1 > q0)
        dq_step<HS, true>(Ks[buf], Vs[buf], key0, qrow, prow, lane, h, c, lse2, Dq, qf, gf, dqa);
      else
        dq_step<HS, false>(Ks[buf], Vs[buf], key0, qrow, prow, lane, h, c, lse2, Dq, qf, gf, dqa);
    }
    if (kt + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  // dQ^T register i of lane (n, h): column d = db*32 + 8*(i/4) + 4h + i%4, query qrow.
  const rsrc_t wq = make_rsrc(dq + base, slice_bytes);
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = uint32_t(qrow * HS + db * 32 + 8 * g + 4 * h) * 2;
      bstore8(wq, off, u32x2{pack_bf16(dqa[db][4 * g] * scale, dqa[db][4 * g + 1] * scale),
                             pack_bf16(dqa[db][4 * g + 2] * scale, dqa[db][4 * g + 3] * scale)});
    }
}

}  // namespace

hipError_t bf16_bwd_pre(const uint16_t* o, const uint16_t* dO, float* D, int BH, int T, int hs,
                        hipStream_t s) {
  const long rows = long(BH) * T;
  const long threads = rows * (hs / 8);
  const dim3 grid(unsigned((threads + kThreads - 1) / kThreads));
  if (hs == 64) return launch(bf16_pre_kernel<64>, grid, dim3(kThreads), s, o, dO, D, rows);
  return launch(bf16_pre_kernel<32>, grid, dim3(kThreads), s, o, dO, D, rows);
}

hipError_t bf16_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, const float* lse, const float* D, uint16_t* dk,
                         uint16_t* dv, int BH, int T, int hs, float scale, hipStream_t s) {
  const int bn = 128;
  const dim3 grid(unsigned(((T + bn - 1) / bn) * BH));
  if (hs == 64)
    return launch(bf16_dkdv_kernel<64>, grid, dim3(kThreads), s, q, k, v, dO, lse, D, dk, dv, BH,
                  T, scale);
  return launch(bf16_dkdv_kernel<32>, grid, dim3(kThreads), s, q, k, v, dO, lse, D, dk, dv, BH, T,
                scale);
}

hipError_t bf16_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint16_t* dO, const float* lse, const float* D, uint16_t* dq, int BH,
                       int T, int hs, float scale, hipStream_t s) {
  const int bm = 128;
  const dim3 grid(unsigned(((T + bm - 1) / bm) * BH));
  if (hs == 64)
    return launch(bf16_dq_kernel<64>, grid, dim3(kThreads), s, q, k, v, dO, lse, D, dq, BH, T,
                  scale);
  return launch(bf16_dq_kernel<32>, grid, dim3(kThreads), s, q, k, v, dO, lse, D, dq, BH, T,
                scale);
}

}  // namespace gattn
