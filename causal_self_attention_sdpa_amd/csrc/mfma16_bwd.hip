// 16-bit (bf16 or fp16) causal attention backward on gfx950 MFMA: two main
// kernels, no atomics; E is the element type's traits.
//
// The pages state only that the model is trained with a backward pass; the
// gradients are the chain rule of the forward ("Let's build GPT" summary
// page: tril mask 48:54 / 55:20, row softmax 51:04, scaled q.k 1:06:16 /
// 1:17:18, weighted values 1:10:15):
//   P  = exp(scale * Q K^T - lse)    recomputed from the forward's lse,
//                                    exactly 0 above the diagonal
//   D  = rowsum(dO * O)
//   dP = dO V^T,   dS = P * (dP - D)
//   dQ = scale * dS K                          (dQ kernel, per query tile; it
//                                               also writes D and lse*log2(e)
//                                               to the workspace)
//   dV = P^T dO,   dK = scale * dS^T Q        (dK/dV kernel, per key tile)
// Splitting dQ from dK/dV costs a second recomputation of S and dP, and in
// exchange removes float32 atomics (which on this chip are executed past the
// per-XCD L2s), the zeroing and conversion passes of an accumulator, and the
// LDS round trip of dS; every output is deterministic.
//
// With dropout (DROP; mask Z = keep / (1 - p) on the weights, philox.h) the
// forward computed O = (P*Z) V, and the chain rule gives
//   dV = (P*Z)^T dO,   dP = Z * (dO V^T),   dS = P * (dP - D)
// with the same D = rowsum(dO * O) (sum_j P Z (dO V^T) = dO . O).  The keep
// decisions are recomputed from each weight's position, not stored.
//
// Both kernels stream tiles into double-buffered, swizzled LDS tiles by LDS
// DMA (no register staging) with one barrier per step: the DMA for step t+1
// runs while step t computes.  Tensors are addressed through Layout strides
// (q, k, v: li; o, dO: lo; dq, dk, dv: lg), and global accesses go through
// buffer resources sized to the span of one (b, h) slice, so rows past T read
// as zero and their stores are dropped.  A query row past T then has zero q and dO rows (and D = lse = 0):
// its P is 1, but its dP, dS and dO are 0, so it adds exactly nothing.
#include <cmath>

#include "mfma16_common.h"
#include "gattn_internal.h"
#include "philox.h"

#ifndef GATTN_DKDV_STAGES
#define GATTN_DKDV_STAGES 2
#endif
#ifndef GATTN_DQ_STAGES
#define GATTN_DQ_STAGES 2
#endif
#ifndef GATTN_DKDV_OCC
#define GATTN_DKDV_OCC 2
#endif
#ifndef GATTN_DQ_OCC
#define GATTN_DQ_OCC 2
#endif
#ifndef GATTN_DKDV_DROP_OCC
#define GATTN_DKDV_DROP_OCC 2
#endif
#ifndef GATTN_DQ_DROP_OCC
#define GATTN_DQ_DROP_OCC 2
#endif

namespace gattn {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// D[i] = sum_d dO[i][d] * O[i][d] and L2[i] = lse[i] * log2(e); HS/8 threads
// per row, 16-byte loads.
template <class E, int HS>
__global__ __launch_bounds__(kThreads) void pre16_kernel(const uint16_t* __restrict__ o,
                                                           const uint16_t* __restrict__ dO,
                                                           const float* __restrict__ lse,
                                                           float* __restrict__ D,
                                                           float* __restrict__ L2, long rows,
                                                           int H, int T, Layout lo) {
  constexpr int TPR = HS / 8;
  const long gid = long(blockIdx.x) * kThreads + threadIdx.x;
  const long row = gid / TPR;
  const int part = int(gid % TPR);
  float s = 0.f;
  if (row < rows) {
    const int bh = int(row / T);
    const int64_t off = slice_offset(lo, bh, H) + (row - long(bh) * T) * lo.st + part * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + off);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s = fmaf(E::lo(a[w]), E::lo(b[w]), s);
      s = fmaf(E::hi(a[w]), E::hi(b[w]), s);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (row < rows && part == 0) {
    D[row] = s;
    L2[row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup = 4 wavefronts = 128 keys of one (b, h); wavefront w
// keeps keys k0 + 32w .. +31 (K, V as MFMA B operands) and their dK^T, dV^T
// accumulators in registers.  Steps walk 64-query tiles from the diagonal to
// T.  Per 32-query block b of a step:
//   A(b): S = Q K^T, dP = dO V^T    C[query][key]; Q, dO rows read from LDS in
//                                   perm_row order, so each lane's registers
//                                   8t..8t+7 are 8 consecutive queries
//   B(b): P, dS (f32, registers) -> 16-bit, exactly the B operand of
//   C(b): dV^T += dO^T P, dK^T += Q^T dS   C[d][key]; dO^T, Q^T via LDS
//                                          transpose reads
// In the steps that meet the diagonal, blocks wholly before this wavefront's
// keys are skipped and the others masked.
//
// Dropout here sees a weight's keep decision in the transposed position: a
// lane holds 8 consecutive queries of one key, while a generator block
// covers 8 consecutive keys of one query.  The 8 lanes n = 8a .. 8a+7 (same
// h) hold keys 8G .. 8G+7 against the same 8 queries I0 .. I0+7, so lane
// 8a + r draws the block of query I0 + r, and the 8 blocks' keep bytes are
// exchanged among the 8 lanes (xor 1, 2, 4); the lane then reads bit r of
// byte e for query I0 + e.
template <int HS>
struct DkdvCfg {
  static constexpr int NW = 4;
  static constexpr int BN = 32 * NW;  // keys per workgroup
  static constexpr int BQ = 64;       // queries per step
  static constexpr int QB = BQ / 32;
  static constexpr int KSTEP = HS / 16;
  static constexpr int DB = HS / 32;
  static constexpr int NS = GATTN_DKDV_STAGES;  // LDS ring depth
  // DMA instructions per wavefront per step: Q and dO tiles, plus one quarter
  // of the lse and D rows each.
  static constexpr int PER = 2 * (BQ * HS / 512) / NW + 2;
  static_assert((BQ * HS / 512) % NW == 0 && BQ % (4 * NW) == 0, "uniform DMA split");
};

template <int HS>
struct DkdvRegs {
  u32x4 kf[HS / 16], vf[HS / 16];
  f32x16 dka[HS / 32], dva[HS / 32];
};

// A(b): S and dP of query block qb.
template <class E, int HS>
__device__ __forceinline__ void dkdv_sdp(const uint16_t* Qb, const uint16_t* Gb, int qb,
                                const LaneOffsets<HS>& L, const DkdvRegs<HS>& R, f32x16& s,
                                f32x16& dp) {
  using C = DkdvCfg<HS>;
  s = f32x16{};
  dp = f32x16{};
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks) {
    s = E::mfma(op_nat<HS>(Qb, L, qb * 32, ks), R.kf[ks], s);
    dp = E::mfma(op_nat<HS>(Gb, L, qb * 32, ks), R.vf[ks], dp);
  }
}

// Lane xor M within each group of 32 lanes (ds_swizzle, bit-mask mode).
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
  return uint32_t(__builtin_amdgcn_ds_swizzle(int(x), (M << 10) | 0x1F));
}

// The keep bytes of the 8 lanes 8a .. 8a+7 (lane 8a + r passes `byte`, r =
// lane & 7): byte e of (lo, hi) as one 64-bit word is lane 8a + e's byte.
// Placement by per-lane shifts and a bit-field insert (no compares).
__device__ __forceinline__ void gather8(uint32_t byte, int r, uint32_t& lo, uint32_t& hi) {
  const uint32_t s1 = 8u * (r & 1), s2 = 8u * (r & 2);  // 0 or 8; 0 or 16
  const uint32_t m4 = 0u - uint32_t((r >> 2) & 1);      // all ones for the upper 4 lanes
  const uint32_t p1 = xor_lane<1>(byte);
  const uint32_t x16 = (byte << s1) | (p1 << (8u - s1));
  const uint32_t p2 = xor_lane<2>(x16);
  const uint32_t x32 = (x16 << s2) | (p2 << (16u - s2));
  const uint32_t p4 = xor_lane<4>(x32);
  lo = (p4 & m4) | (x32 & ~m4);
  hi = (x32 & m4) | (p4 & ~m4);
}

// Keep bits of this lane's two runs of 8 queries in query block qb (run t:
// queries qs0 + 32 qb + 16 t + 8h + e): bit 8e of w[t][0] (e < 4) or of
// w[t][1] (e >= 4) is the decision for query e of the run and key krow.
__device__ __forceinline__ void dkdv_keep(int qs0, int qb, int krow, int h, uint32_t bh,
                                          const Dropout& dr, uint32_t (&w)[2][2]) {
  const int r = krow & 7;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int q = qs0 + qb * 32 + 16 * t + 8 * h + r;
    gather8(keep_bits8(uint32_t(q), uint32_t(krow) >> 3, bh, dr), r, w[t][0], w[t][1]);
    w[t][0] >>= r;
    w[t][1] >>= r;
  }
}

// B(b) then C(b) for query block qb; w: its keep bits (DROP).
template <class E, int HS, bool MASK, bool DROP>
__device__ __forceinline__ void dkdv_grad(const uint16_t* Qb, const uint16_t* Gb, const float* Lb,
                                 const float* Db, int qb, int qs0, int krow, int h, float c,
                                 const LaneOffsets<HS>& L, const f32x16& s, const f32x16& dp,
                                 DkdvRegs<HS>& R, const uint32_t (&w)[2][2], float zs) {
  using C = DkdvCfg<HS>;
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
      if constexpr (DROP) {
        const uint32_t m = keep_mask(w[t][e >> 2], 8 * (e & 3));
        pv[e] = __uint_as_float(__float_as_uint(p) & m);
        dsv[e] = p * (__uint_as_float(__float_as_uint(dp[8 * t + e] * zs) & m) - De);
      } else {
        pv[e] = p;
        dsv[e] = p * (dp[8 * t + e] - De);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pp[t][e] = E::pack(pv[2 * e], pv[2 * e + 1]);
      dsp[t][e] = E::pack(dsv[2 * e], dsv[2 * e + 1]);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int k0 = qb * 32 + 16 * t;
      R.dva[db] = E::mfma(op_tr<HS>(Gb, L, k0, db), pp[t], R.dva[db]);
      R.dka[db] = E::mfma(op_tr<HS>(Qb, L, k0, db), dsp[t], R.dka[db]);
    }
}

// One step below the diagonal: every block is visible, no mask.
template <class E, int HS, bool DROP>
__device__ __forceinline__ void dkdv_step_full(const uint16_t* Qb, const uint16_t* Gb, const float* Lb,
                                      const float* Db, int qs0, int krow, int h, float c,
                                      const LaneOffsets<HS>& L, DkdvRegs<HS>& R, uint32_t bh,
                                      const Dropout& dr) {
  using C = DkdvCfg<HS>;
  if constexpr (DROP) {  // block by block: the generator's registers leave no room for both
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      uint32_t w[2][2] = {};
      dkdv_keep(qs0, qb, krow, h, bh, dr, w);
      f32x16 s, dp;
      dkdv_sdp<E, HS>(Qb, Gb, qb, L, R, s, dp);
      dkdv_grad<E, HS, false, DROP>(Qb, Gb, Lb, Db, qb, qs0, krow, h, c, L, s, dp, R, w, dr.zs);
    }
  } else {
    // S and dP of both blocks first: block 1's MFMAs run while block 0's
    // weights and dS are computed on the vector ALU.
    static_assert(C::QB == 2, "two query blocks per step");
    const uint32_t w[2][2] = {};
    f32x16 s0, dp0, s1, dp1;
    dkdv_sdp<E, HS>(Qb, Gb, 0, L, R, s0, dp0);
    dkdv_sdp<E, HS>(Qb, Gb, 1, L, R, s1, dp1);
    dkdv_grad<E, HS, false, DROP>(Qb, Gb, Lb, Db, 0, qs0, krow, h, c, L, s0, dp0, R, w, dr.zs);
    dkdv_grad<E, HS, false, DROP>(Qb, Gb, Lb, Db, 1, qs0, krow, h, c, L, s1, dp1, R, w, dr.zs);
  }
}

// A step that meets the diagonal: blocks wholly before this wavefront's keys
// are skipped, the others masked.
template <class E, int HS, bool DROP>
__device__ __forceinline__ void dkdv_step_diag(const uint16_t* Qb, const uint16_t* Gb, const float* Lb,
                                      const float* Db, int qs0, int kw0, int krow, int h, float c,
                                      const LaneOffsets<HS>& L, DkdvRegs<HS>& R, uint32_t bh,
                                      const Dropout& dr) {
  using C = DkdvCfg<HS>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    if (kw0 > qs0 + qb * 32 + 31) continue;  // all of this wavefront's keys lie after the block
    uint32_t w[2][2] = {};
    if constexpr (DROP) dkdv_keep(qs0, qb, krow, h, bh, dr, w);
    f32x16 s, dp;
    dkdv_sdp<E, HS>(Qb, Gb, qb, L, R, s, dp);
    dkdv_grad<E, HS, true, DROP>(Qb, Gb, Lb, Db, qb, qs0, krow, h, c, L, s, dp, R, w, dr.zs);
  }
}

// STRIDED = false: every tensor is contiguous (B, H, T, hs) and the row
// strides are the compile-time HS (the strides' registers and multiplies
// would otherwise push this kernel into spills).  DROP: dropout with dr.
template <class E, int HS, bool STRIDED, bool DROP>
__global__ __launch_bounds__(kThreads, DROP ? GATTN_DKDV_DROP_OCC : GATTN_DKDV_OCC) void dkdv16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ Dg, const float* __restrict__ L2g, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int BH, int H, int T, float scale, Layout li, Layout lo,
    Layout lg, Dropout dr) {
  using C = DkdvCfg<HS>;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[C::NS][C::BQ * HS];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[C::NS][C::BQ * HS];
  __shared__ __attribute__((aligned(16))) float Ls[C::NS][C::BQ];
  __shared__ __attribute__((aligned(16))) float Ds[C::NS][C::BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  // Key tiles near the start have the most query tiles below the diagonal.
  const int kt = int(blockIdx.x) / BH;
  const int bh = int(blockIdx.x) % BH;
  const int64_t base = slice_base<HS, STRIDED>(li, bh, H, T);
  const uint32_t slice_bytes = slice_bytes_of<HS, STRIDED>(li, T);
  const int rs = STRIDED ? int(li.st) : HS, rso = STRIDED ? int(lo.st) : HS;
  const rsrc_t rq = make_rsrc(q + base, slice_bytes), rk = make_rsrc(k + base, slice_bytes);
  const rsrc_t rv = make_rsrc(v + base, slice_bytes);
  const rsrc_t rg = make_rsrc(dO + slice_base<HS, STRIDED>(lo, bh, H, T),
                              slice_bytes_of<HS, STRIDED>(lo, T));
  const rsrc_t rl = make_rsrc(L2g + long(bh) * T, uint32_t(T) * 4);
  const rsrc_t rd = make_rsrc(Dg + long(bh) * T, uint32_t(T) * 4);

  const int k0 = kt * C::BN;
  const int kw0 = k0 + 32 * w;
  const int krow = kw0 + n;
  const float c = scale * kLog2e;

  DkdvRegs<HS> R;
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks) {
    const uint32_t off = uint32_t(krow * rs + 16 * ks + 8 * h) * 2;
    R.kf[ks] = bload16(rk, off);
    R.vf[ks] = bload16(rv, off);
  }
#pragma unroll
  for (int db = 0; db < C::DB; ++db) R.dka[db] = R.dva[db] = f32x16{};

  constexpr int QQ = C::BQ / C::NW;  // lse / D rows per wavefront
  auto issue = [&](int qt, int buf) {
    dma_tile<HS, C::BQ, C::NW>(rq, qt * C::BQ, rs, Qs[buf], w, lane);
    dma_tile<HS, C::BQ, C::NW>(rg, qt * C::BQ, rso, Gs[buf], w, lane);
    const uint32_t off = uint32_t(qt * C::BQ + w * QQ) * 4;
    dma_f32(rl, off, Ls[buf] + w * QQ, QQ, lane);
    dma_f32(rd, off, Ds[buf] + w * QQ, QQ, lane);
  };

  const int nqt = (T + C::BQ - 1) / C::BQ;
  const int qt0 = k0 / C::BQ;
  const int nsteps = nqt - qt0;
  const LaneOffsets<HS> L(lane);
#pragma unroll
  for (int j = 0; j < C::NS - 1; ++j)
    if (j < nsteps) issue(qt0 + j, j);
  wait_ring<C::NS, C::PER>(min(C::NS - 2, nsteps - 1));
  __syncthreads();
  // One step: prefetch step t+NS-1 into the buffer freed by step t-1, compute
  // step t, wait until step t+1 has landed, publish.
  auto step = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (t + C::NS - 1 < nsteps) issue(qt0 + t + C::NS - 1, (buf + C::NS - 1) % C::NS);
    const int qs0 = (qt0 + t) * C::BQ;
    if (qs0 < k0 + C::BN)
      dkdv_step_diag<E, HS, DROP>(Qs[buf], Gs[buf], Ls[buf], Ds[buf], qs0, kw0, krow, h, c, L, R,
                                  uint32_t(bh), dr);
    else
      dkdv_step_full<E, HS, DROP>(Qs[buf], Gs[buf], Ls[buf], Ds[buf], qs0, krow, h, c, L, R,
                                  uint32_t(bh), dr);
    wait_ring<C::NS, C::PER>(max(0, min(C::NS - 2, nsteps - t - 2)));
    __syncthreads();
  };
  ring_loop<C::NS>(nsteps, step);

  // dK^T / dV^T register i of lane (n, h): column d = db*32 + 8*(i/4) + 4h + i%4, key krow.
  const int64_t gbase = slice_base<HS, STRIDED>(lg, bh, H, T);
  const uint32_t gbytes = slice_bytes_of<HS, STRIDED>(lg, T);
  const rsrc_t wk = make_rsrc(dk + gbase, gbytes), wv = make_rsrc(dv + gbase, gbytes);
  const int rsg = STRIDED ? int(lg.st) : HS;
  const float zv = DROP ? dr.zs : 1.f;  // dV = (P*Z)^T dO: the kept weights' factor
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = uint32_t(krow * rsg + db * 32 + 8 * g + 4 * h) * 2;
      bstore8(wv, off, u32x2{E::pack(R.dva[db][4 * g] * zv, R.dva[db][4 * g + 1] * zv),
                             E::pack(R.dva[db][4 * g + 2] * zv, R.dva[db][4 * g + 3] * zv)});
      bstore8(wk, off, u32x2{E::pack(R.dka[db][4 * g] * scale, R.dka[db][4 * g + 1] * scale),
                             E::pack(R.dka[db][4 * g + 2] * scale, R.dka[db][4 * g + 3] * scale)});
    }
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 4 wavefronts = 128 queries of one (b, h); wavefront w keeps
// queries r0 + 32w .. +31 (Q^T and dO^T as MFMA B operands, lse and D as
// per-lane scalars) and the dQ^T accumulator in registers.  It computes D
// from its O and dO rows and writes D and lse*log2(e) to the workspace for
// the dK/dV kernel.  Steps walk 64-key tiles from 0 to the diagonal.  Per
// step and 32-key block:
//   S^T = K Q^T, dP^T = V dO^T      C[key][query]; K, V rows from LDS in
//                                   perm_row order (8 consecutive keys per
//                                   lane in registers 8t..8t+7)
//   dS^T (f32) -> 16-bit             the B operand of
//   dQ^T += K^T dS^T                 C[d][query]; K^T via LDS transpose reads
template <int HS>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int BM = 32 * NW;  // queries per workgroup
  static constexpr int BN = 64;       // keys per step
  static constexpr int KSTEP = HS / 16;
  static constexpr int DB = HS / 32;
  static constexpr int NS = GATTN_DQ_STAGES;  // LDS ring depth
  static constexpr int PER = 2 * (BN * HS / 512) / NW;  // DMA instructions per wavefront per step
  static_assert((BN * HS / 512) % NW == 0, "uniform DMA split");
};

// Kinds of key tile for one wavefront (32 queries q0 .. q0+31, 64 keys from
// key0, q0 - key0 a multiple of 32): kFull, every key <= every query;
// kDiagLo, key0 == q0: the first 32 keys form the diagonal block, the other
// 32 lie after every query (skipped); kDiagHi, key0 + 32 == q0: the second
// 32 keys form the diagonal block.  In the diagonal block register 8t+e of
// lane (n, h) holds key (q0 + 16t + 8h + e), after query q0 + n exactly when
// 16t + e > dn = n - 8h.  With DROP, registers 8t..8t+7 of block kb are keys
// 8 * (g0 + 4 kb + 2 t) .. +7 of query qrow (g0 = key0 / 8 + h): one generator
// block, as in the forward.
enum DqTile { kFull = 0, kDiagLo = 1, kDiagHi = 2 };

template <class E, int HS, int KIND, bool DROP>
__device__ __forceinline__ void dq_step(const uint16_t* Kb, const uint16_t* Vb, int dn, float c,
                                        float lse2, float Dq, const LaneOffsets<HS>& L,
                                        const u32x4 (&qf)[HS / 16], const u32x4 (&gf)[HS / 16],
                                        f32x16 (&dqa)[HS / 32], uint32_t qrow, uint32_t g0,
                                        uint32_t bh, const Dropout& dr) {
  using C = DqCfg<HS>;
  constexpr int NKB = KIND == kDiagLo ? 1 : 2;  // 32-key blocks computed
  constexpr int KD = KIND == kDiagLo ? 0 : (KIND == kDiagHi ? 1 : -1);  // the diagonal block
  u32x4 dsp[2][2];
  // Keep bits of the step's runs, drawn before the S / dP MFMAs so that the
  // generator's vector ALU work overlaps them.
  uint32_t bits[2][2] = {{0xFFu, 0xFFu}, {0xFFu, 0xFFu}};
  if constexpr (DROP) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) bits[kb][t] = keep_bits8(qrow, g0 + 4 * kb + 2 * t, bh, dr);
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    f32x16 st = {}, dpt = {};
#pragma unroll
    for (int ks = 0; ks < C::KSTEP; ++ks) {
      st = E::mfma(op_nat<HS>(Kb, L, kb * 32, ks), qf[ks], st);
      dpt = E::mfma(op_nat<HS>(Vb, L, kb * 32, ks), gf[ks], dpt);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float p = __builtin_amdgcn_exp2f(fmaf(st[8 * t + e], c, -lse2));
        if (kb == KD && 16 * t + e > dn) p = 0.f;
        if constexpr (DROP)
          dsv[e] = p * (keep_or_zero(dpt[8 * t + e] * dr.zs, bits[kb][t], e) - Dq);
        else
          dsv[e] = p * (dpt[8 * t + e] - Dq);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dsp[kb][t][e] = E::pack(dsv[2 * e], dsv[2 * e + 1]);
    }
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        dqa[db] = E::mfma(op_tr<HS>(Kb, L, kb * 32 + 16 * t, db), dsp[kb][t], dqa[db]);
  // Scheduling hint: spread the MFMAs over the step, each followed by vector
  // ALU work and LDS reads of other blocks, instead of phase after phase.
#pragma unroll
  for (int i = 0; i < NKB * (2 * C::KSTEP + 2 * C::DB); ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

template <class E, int HS, bool STRIDED, bool DROP>  // STRIDED, DROP as for the dK/dV kernel
__global__ __launch_bounds__(kThreads, DROP ? GATTN_DQ_DROP_OCC : GATTN_DQ_OCC) void dq16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, float* __restrict__ Dg,
    float* __restrict__ L2g, uint16_t* __restrict__ dq, int BH, int H, int T, float scale,
    Layout li, Layout lo, Layout lg, Dropout dr) {
  using C = DqCfg<HS>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[C::NS][C::BN * HS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[C::NS][C::BN * HS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int nqt = (T + C::BM - 1) / C::BM;
  const int qt = nqt - 1 - int(blockIdx.x) / BH;  // heaviest query tiles first
  const int bh = int(blockIdx.x) % BH;
  const int64_t base = slice_base<HS, STRIDED>(li, bh, H, T);
  const uint32_t slice_bytes = slice_bytes_of<HS, STRIDED>(li, T);
  const int rs = STRIDED ? int(li.st) : HS, rso = STRIDED ? int(lo.st) : HS;
  const rsrc_t rq = make_rsrc(q + base, slice_bytes), rk = make_rsrc(k + base, slice_bytes);
  const rsrc_t rv = make_rsrc(v + base, slice_bytes);
  const int64_t obase = slice_base<HS, STRIDED>(lo, bh, H, T);
  const uint32_t obytes = slice_bytes_of<HS, STRIDED>(lo, T);
  const rsrc_t rg = make_rsrc(dO + obase, obytes), ro = make_rsrc(o + obase, obytes);

  const int r0 = qt * C::BM;
  const int q0 = r0 + 32 * w;
  const int qrow = q0 + n;
  const int dn = n - 8 * h;
  const float c = scale * kLog2e;

  auto issue = [&](int kt, int buf) {
    dma_tile<HS, C::BN, C::NW>(rk, kt * C::BN, rs, Ks[buf], w, lane);
    dma_tile<HS, C::BN, C::NW>(rv, kt * C::BN, rs, Vs[buf], w, lane);
  };
  const int nkt = (min(r0 + C::BM, T) - 1) / C::BN + 1;
#pragma unroll
  for (int j = 0; j < C::NS - 1; ++j)
    if (j < nkt) issue(j, j);

  // Q^T, dO^T fragments (lane (n, h): row qrow, columns 16 ks + 8h .. +7), and
  // D = rowsum(dO * O) of this lane's query from the same columns of O.
  u32x4 qf[C::KSTEP], gf[C::KSTEP];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks) {
    const uint32_t col = uint32_t(16 * ks + 8 * h);
    qf[ks] = bload16(rq, (uint32_t(qrow * rs) + col) * 2);
    const uint32_t offo = (uint32_t(qrow * rso) + col) * 2;
    gf[ks] = bload16(rg, offo);
    const u32x4 of = bload16(ro, offo);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dpart = fmaf(E::lo(of[e]), E::lo(gf[ks][e]), dpart);
      dpart = fmaf(E::hi(of[e]), E::hi(gf[ks][e]), dpart);
    }
  }
  const float Dq = halves_sum(dpart);
  const float lse2 = bloadf(make_rsrc(lse + long(bh) * T, uint32_t(T) * 4), uint32_t(qrow) * 4) *
                     kLog2e;
  if (h == 0) {
    bstoref(make_rsrc(Dg + long(bh) * T, uint32_t(T) * 4), uint32_t(qrow) * 4, Dq);
    bstoref(make_rsrc(L2g + long(bh) * T, uint32_t(T) * 4), uint32_t(qrow) * 4, lse2);
  }
  f32x16 dqa[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dqa[db] = f32x16{};

  const LaneOffsets<HS> L(lane);
  wait_vmem();  // the first tile and this wavefront's q, dO, O, lse rows
  __syncthreads();
  // One step: prefetch key tile kt+NS-1 into the buffer freed by tile kt-1,
  // compute tile kt, wait until tile kt+1 has landed, publish.
  auto step = [&](int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (kt + C::NS - 1 < nkt) issue(kt + C::NS - 1, (buf + C::NS - 1) % C::NS);
    const int key0 = kt * C::BN;
    const uint32_t g0 = uint32_t(key0 / 8 + h), ub = uint32_t(bh), uq = uint32_t(qrow);
    if (q0 < T && key0 <= q0) {
      if (key0 == q0)
        dq_step<E, HS, kDiagLo, DROP>(Ks[buf], Vs[buf], dn, c, lse2, Dq, L, qf, gf, dqa, uq, g0,
                                      ub, dr);
      else if (key0 + 32 == q0)
        dq_step<E, HS, kDiagHi, DROP>(Ks[buf], Vs[buf], dn, c, lse2, Dq, L, qf, gf, dqa, uq, g0,
                                      ub, dr);
      else
        dq_step<E, HS, kFull, DROP>(Ks[buf], Vs[buf], dn, c, lse2, Dq, L, qf, gf, dqa, uq, g0, ub,
                                    dr);
    }
    wait_ring<C::NS, C::PER>(max(0, min(C::NS - 2, nkt - kt - 2)));
    __syncthreads();
  };
  ring_loop<C::NS>(nkt, step);

  // dQ^T register i of lane (n, h): column d = db*32 + 8*(i/4) + 4h + i%4, query qrow.
  const rsrc_t wq = make_rsrc(dq + slice_base<HS, STRIDED>(lg, bh, H, T),
                              slice_bytes_of<HS, STRIDED>(lg, T));
  const int rsg = STRIDED ? int(lg.st) : HS;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = uint32_t(qrow * rsg + db * 32 + 8 * g + 4 * h) * 2;
      bstore8(wq, off, u32x2{E::pack(dqa[db][4 * g] * scale, dqa[db][4 * g + 1] * scale),
                             E::pack(dqa[db][4 * g + 2] * scale, dqa[db][4 * g + 3] * scale)});
    }
}

}  // namespace

namespace {
template <class E>
hipError_t pre16_launch(const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                        float* L2, int BH, int H, int T, int hs, Layout lo, hipStream_t s) {
  const long rows = long(BH) * T;
  const long threads = rows * (hs / 8);
  const dim3 grid(unsigned((threads + kThreads - 1) / kThreads));
  auto kern = hs == 64 ? pre16_kernel<E, 64> : pre16_kernel<E, 32>;
  return launch(kern, grid, dim3(kThreads), s, o, dO, lse, D, L2, rows, H, T, lo);
}

template <class E>
hipError_t dkdv16_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, const float* D, const float* L2, uint16_t* dk,
                         uint16_t* dv, int BH, int H, int T, int hs, float scale, Layout li,
                         Layout lo, Layout lg, const Dropout& dr, hipStream_t s) {
  const int bn = DkdvCfg<64>::BN;
  const dim3 grid(unsigned(((T + bn - 1) / bn) * BH));
  const bool strided = !all_contiguous(H, T, hs, li, lo, lg);
  auto pick = [&](auto dropc) {
    constexpr bool D = decltype(dropc)::value;
    return hs == 64 ? (strided ? dkdv16_kernel<E, 64, true, D> : dkdv16_kernel<E, 64, false, D>)
                    : (strided ? dkdv16_kernel<E, 32, true, D> : dkdv16_kernel<E, 32, false, D>);
  };
  auto kern = dr.thr != 0 ? pick(std::true_type{}) : pick(std::false_type{});
  return launch(kern, grid, dim3(kThreads), s, q, k, v, dO, D, L2, dk, dv, BH, H, T, scale, li, lo,
                lg, dr);
}

template <class E>
hipError_t dq16_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                       float* L2, uint16_t* dq, int BH, int H, int T, int hs, float scale,
                       Layout li, Layout lo, Layout lg, const Dropout& dr, hipStream_t s) {
  const int bm = DqCfg<64>::BM;
  const dim3 grid(unsigned(((T + bm - 1) / bm) * BH));
  const bool strided = !all_contiguous(H, T, hs, li, lo, lg);
  auto pick = [&](auto dropc) {
    constexpr bool D = decltype(dropc)::value;
    return hs == 64 ? (strided ? dq16_kernel<E, 64, true, D> : dq16_kernel<E, 64, false, D>)
                    : (strided ? dq16_kernel<E, 32, true, D> : dq16_kernel<E, 32, false, D>);
  };
  auto kern = dr.thr != 0 ? pick(std::true_type{}) : pick(std::false_type{});
  return launch(kern, grid, dim3(kThreads), s, q, k, v, o, dO, lse, D, L2, dq, BH, H, T, scale, li,
                lo, lg, dr);
}
}  // namespace

hipError_t h16_bwd_pre(const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                       float* L2, int BH, int H, int T, int hs, Layout lo, bool f16,
                       hipStream_t s) {
  if (f16) return pre16_launch<F16>(o, dO, lse, D, L2, BH, H, T, hs, lo, s);
  return pre16_launch<Bf16>(o, dO, lse, D, L2, BH, H, T, hs, lo, s);
}

hipError_t h16_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* dO, const float* D, const float* L2, uint16_t* dk,
                        uint16_t* dv, int BH, int H, int T, int hs, float scale, Layout li,
                        Layout lo, Layout lg, const Dropout& dr, bool f16, hipStream_t s) {
  if (f16)
    return dkdv16_launch<F16>(q, k, v, dO, D, L2, dk, dv, BH, H, T, hs, scale, li, lo, lg, dr, s);
  return dkdv16_launch<Bf16>(q, k, v, dO, D, L2, dk, dv, BH, H, T, hs, scale, li, lo, lg, dr, s);
}

hipError_t h16_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                      float* L2, uint16_t* dq, int BH, int H, int T, int hs, float scale,
                      Layout li, Layout lo, Layout lg, const Dropout& dr, bool f16,
                      hipStream_t s) {
  if (f16)
    return dq16_launch<F16>(q, k, v, o, dO, lse, D, L2, dq, BH, H, T, hs, scale, li, lo, lg, dr, s);
  return dq16_launch<Bf16>(q, k, v, o, dO, lse, D, L2, dq, BH, H, T, hs, scale, li, lo, lg, dr, s);
}

}  // namespace gattn
