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
// decisions come as bits: stored by the forward, or drawn once by the dQ
// kernel from each weight's position and stored for the dK/dV kernel.  The
// kept weights' factor zs is folded into the exponent (pz = P zs =
// 2^(s c - (L2 - log2 zs))), so with the row terms D z = D / zs a weight's
// dS = pz (keep ? dP - D z : -D z) and its dV weight pz keep; with dropout
// the workspace holds L2 - log2 zs and D / zs for the dK/dV kernel.
//
// Both kernels stream tiles into swizzled LDS rings by LDS DMA (no register
// staging) with one barrier per step, so the DMA of later steps runs while a
// step computes (two stages for dK/dV, three for dQ, whose K tile is also
// converted to fp16 one step ahead).  Tensors are addressed through Layout strides
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
// S and dK use fp16 operands (see DsOf): the Q tile is converted in place as
// it lands, the K fragments once; dP and dV stay in the input type.  D is
// the exact row term the dQ kernel wrote.
// In the steps that meet the diagonal, blocks wholly before this wavefront's
// keys are skipped and the others masked.
//
// With dropout the keep decisions are not drawn here: the dQ kernel, which
// runs first and draws every decision of the causal pairs (one generator
// block = 8 consecutive keys of one query), stores them in the workspace as
// 8x8 blocks: block (query octet I, key group G) is 8 bytes at
// ((I * ng + G) * 8) of the slice's part (ng = ceil(T / 8)), byte e holding
// query 8I + e's bits, bit r key 8G + r.  Each step DMAs the 8 x 16 blocks of
// its 64 queries and the workgroup's 128 keys into LDS next to the Q and dO
// tiles; a lane (8 consecutive queries of one key per run) reads one block
// per run and bit r of byte e.
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
  // of the lse and D rows each (with dropout, one more: a quarter of the
  // step's keep-bit blocks).
  static constexpr int PER = 2 * (BQ * HS / 512) / NW + 2;
  static constexpr int KEEP_WORDS = (BQ / 8) * (BN / 8) * 2;  // keep-bit tile, 32-bit words
  static_assert((BQ * HS / 512) % NW == 0 && BQ % (4 * NW) == 0, "uniform DMA split");
};

// kf, vf: the lane's K and V fragments (B operands of A(b)), held in
// registers in the contiguous kernel without dropout; with dropout or
// strided layouts they are read from the workgroup's K and V tiles in LDS
// for each block instead (KVb: K tile, then V tile), which leaves the
// registers the masks or the strides need.
template <int HS>
struct DkdvRegs {
  u32x4 kf[HS / 16], vf[HS / 16];
  f32x16 dka[HS / 32], dva[HS / 32];
};

// A(b): S and dP of query block qb.  kl: the lane's key row in the
// workgroup's tiles.
template <class E, int HS, bool KVL>
__device__ __forceinline__ void dkdv_sdp(const uint16_t* Qb, const uint16_t* Gb,
                                const uint16_t* KVb, int kl, int h, int qb,
                                const LaneOffsets<HS>& L, const DkdvRegs<HS>& R, f32x16& s,
                                f32x16& dp) {
  using C = DkdvCfg<HS>;
  s = f32x16{};
  dp = f32x16{};
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks) {
    const u32x4 kf = KVL ? tile_row16<HS>(KVb, kl, 16 * ks + 8 * h) : R.kf[ks];
    const u32x4 vf = KVL ? tile_row16<HS>(KVb + C::BN * HS, kl, 16 * ks + 8 * h) : R.vf[ks];
    s = DsOf<E>::T::mfma(op_nat<HS>(Qb, L, qb * 32, ks), kf, s);
    dp = E::mfma(op_nat<HS>(Gb, L, qb * 32, ks), vf, dp);
  }
}

// Keep bits of this lane's run t of 8 queries in query block qb (queries
// qs0 + 32 qb + 16 t + 8h + e) for its key, from the step's keep-bit tile Bb
// (block of query octet a, key group gl at words 2 (16 a + gl) and +1);
// r = key & 7.  Bit 8e of w[0] (e < 4) or of w[1] (e >= 4) is then the
// decision for query e of the run.
__device__ __forceinline__ u32x2 dkdv_keep(const uint32_t* Bb, int qb, int t, int h, int gl,
                                           int r) {
  const u32x2 blk = *reinterpret_cast<const u32x2*>(Bb + 2 * (16 * (4 * qb + 2 * t + h) + gl));
  return u32x2{blk[0] >> r, blk[1] >> r};
}

// B(b) then C(b) for query block qb; with DROP, the keep bits come from the
// step's keep-bit tile Bb (this lane's key group gl), read run by run.
template <class E, int HS, bool MASK, bool DROP>
__device__ __forceinline__ void dkdv_grad(const uint16_t* Qb, const uint16_t* Gb, const float* Lb,
                                 const float* Db, const uint32_t* Bb, int qb, int qs0, int krow,
                                 int h, float c, const LaneOffsets<HS>& L, const f32x16& s,
                                 const f32x16& dp, DkdvRegs<HS>& R, int gl) {
  using C = DkdvCfg<HS>;
  u32x4 pp[2], dsp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int ql = qb * 32 + 16 * t + 8 * h;  // local index of this lane's run of 8 queries
    u32x2 w = {};
    if constexpr (DROP) w = dkdv_keep(Bb, qb, t, h, gl, krow & 7);
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
        const uint32_t m = keep_mask(w[e >> 2], 8 * (e & 3));
        pv[e] = __uint_as_float(__float_as_uint(p) & m);  // p is P zs, De is D / zs
        dsv[e] = p * (__uint_as_float(__float_as_uint(dp[8 * t + e]) & m) - De);
      } else {
        pv[e] = p;
        dsv[e] = p * (dp[8 * t + e] - De);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pp[t][e] = E::pack(pv[2 * e], pv[2 * e + 1]);
      dsp[t][e] = DsOf<E>::T::pack(dsv[2 * e], dsv[2 * e + 1]);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int k0 = qb * 32 + 16 * t;
      R.dva[db] = E::mfma(op_tr<HS>(Gb, L, k0, db), pp[t], R.dva[db]);
      R.dka[db] = DsOf<E>::T::mfma(op_tr<HS>(Qb, L, k0, db), dsp[t], R.dka[db]);
    }
}

// One step below the diagonal: every block is visible, no mask.  S and dP of
// both blocks first: block 1's MFMAs run while block 0's weights and dS are
// computed on the vector ALU.
template <class E, int HS, bool DROP, bool KVL>
__device__ __forceinline__ void dkdv_step_full(const uint16_t* Qb, const uint16_t* Gb, const float* Lb,
                                      const float* Db, const uint32_t* Bb, const uint16_t* KVb,
                                      int kl, int qs0, int krow, int h, float c,
                                      const LaneOffsets<HS>& L, DkdvRegs<HS>& R, int gl) {
  using C = DkdvCfg<HS>;
  static_assert(C::QB == 2, "two query blocks per step");
  f32x16 s0, dp0, s1, dp1;
  dkdv_sdp<E, HS, KVL>(Qb, Gb, KVb, kl, h, 0, L, R, s0, dp0);
  dkdv_sdp<E, HS, KVL>(Qb, Gb, KVb, kl, h, 1, L, R, s1, dp1);
  dkdv_grad<E, HS, false, DROP>(Qb, Gb, Lb, Db, Bb, 0, qs0, krow, h, c, L, s0, dp0, R, gl);
  dkdv_grad<E, HS, false, DROP>(Qb, Gb, Lb, Db, Bb, 1, qs0, krow, h, c, L, s1, dp1, R, gl);
}

// A step that meets the diagonal: blocks wholly before this wavefront's keys
// are skipped, the others masked.
template <class E, int HS, bool DROP, bool KVL>
__device__ __forceinline__ void dkdv_step_diag(const uint16_t* Qb, const uint16_t* Gb, const float* Lb,
                                      const float* Db, const uint32_t* Bb, const uint16_t* KVb,
                                      int kl, int qs0, int kw0, int krow, int h, float c,
                                      const LaneOffsets<HS>& L, DkdvRegs<HS>& R, int gl) {
  using C = DkdvCfg<HS>;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    if (kw0 > qs0 + qb * 32 + 31) continue;  // all of this wavefront's keys lie after the block
    f32x16 s, dp;
    dkdv_sdp<E, HS, KVL>(Qb, Gb, KVb, kl, h, qb, L, R, s, dp);
    dkdv_grad<E, HS, true, DROP>(Qb, Gb, Lb, Db, Bb, qb, qs0, krow, h, c, L, s, dp, R, gl);
  }
}

// STRIDED = false: every tensor is contiguous (B, H, T, hs) and the row
// strides are the compile-time HS (the strides' registers and multiplies
// would otherwise push this kernel into spills).  DROP: dropout with dr.
template <class E, int HS, bool STRIDED, bool DROP>
__global__ __launch_bounds__(kThreads, DROP ? GATTN_DKDV_DROP_OCC : GATTN_DKDV_OCC) void dkdv16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ Dg, const float* __restrict__ L2g,
    const uint64_t* __restrict__ keep, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    int BH, int H, int T, float scale, Layout li, Layout lo, Layout lg, Dropout dr) {
  using C = DkdvCfg<HS>;
  constexpr int PER = C::PER + (DROP ? 1 : 0);
  constexpr bool KVL = DROP || STRIDED;  // K, V fragments from LDS tiles
  __shared__ __attribute__((aligned(16))) uint16_t Qs[C::NS][C::BQ * HS];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[C::NS][C::BQ * HS];
  __shared__ __attribute__((aligned(16))) float Ls[C::NS][C::BQ];
  __shared__ __attribute__((aligned(16))) float Ds[C::NS][C::BQ];
  __shared__ __attribute__((aligned(16))) uint32_t Bs[DROP ? C::NS : 1][DROP ? C::KEEP_WORDS : 4];
  __shared__ __attribute__((aligned(16))) uint16_t KVs[KVL ? 2 * C::BN * HS : 8];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  // Key tiles near the start have the most query tiles below the diagonal.
  const int BH8 = heads_padded(BH);
  const int kt = int(blockIdx.x) / BH8;
  const int bh = int(blockIdx.x) % BH8;
  if (bh >= BH) return;  // grid padding (uniform in the workgroup, before any barrier)
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
  // Keep bits (DROP): this slice's ng x ng blocks of 8 bytes; gl = this
  // lane's key group within the workgroup's 16.
  const uint32_t ng = uint32_t(T + 7) >> 3;
  const rsrc_t rb = make_rsrc(DROP ? keep + int64_t(bh) * ng * ng : keep, ng * ng * 8);
  const int gl = (krow - k0) >> 3;

  DkdvRegs<HS> R;
  if constexpr (KVL) {
    dma_tile<HS, C::BN, C::NW>(rk, k0, rs, KVs, w, lane);
    dma_tile<HS, C::BN, C::NW>(rv, k0, rs, KVs + C::BN * HS, w, lane);
  } else {
#pragma unroll
    for (int ks = 0; ks < C::KSTEP; ++ks) {
      const uint32_t off = uint32_t(krow * rs + 16 * ks + 8 * h) * 2;
      R.kf[ks] = bload16(rk, off);
      R.vf[ks] = bload16(rv, off);
    }
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
    if constexpr (DROP) {
      // Wavefront w: query octets 2w, 2w+1 of the step, 16 key groups each
      // (lane: octet 2w + lane/8, groups 2 (lane%8) and +1; 16 bytes).
      constexpr int KQ = C::KEEP_WORDS / C::NW;  // words per wavefront
      const uint32_t qo = uint32_t(qt * (C::BQ / 8) + 2 * w + (lane >> 3));
      if (lane < 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(Bs[buf] + w * KQ), 16,
            (qo * ng + uint32_t(k0 >> 3) + 2u * uint32_t(lane & 7)) * 8, 0, 0, 0);
    }
  };

  const int nqt = (T + C::BQ - 1) / C::BQ;
  const int qt0 = k0 / C::BQ;
  const int nsteps = nqt - qt0;
  const LaneOffsets<HS> L(lane);
#pragma unroll
  for (int j = 0; j < C::NS - 1; ++j)
    if (j < nsteps) issue(qt0 + j, j);
  wait_ring<C::NS, PER>(min(C::NS - 2, nsteps - 1));  // also the K, V fragments or tiles
  if constexpr (DsOf<E>::kConvert) {
    if constexpr (KVL) {
      dma_tile_to_f16<HS, C::BN, C::NW>(KVs, w, lane);
    } else {
#pragma unroll
      for (int ks = 0; ks < C::KSTEP; ++ks) R.kf[ks] = bf16x8_to_f16x8(R.kf[ks]);
    }
    dma_tile_to_f16<HS, C::BQ, C::NW>(Qs[0], w, lane);
  }
  __syncthreads();
  // One step: prefetch step t+NS-1 into the buffer freed by step t-1, compute
  // step t, wait until step t+1 has landed, convert this wavefront's part of
  // its Q tile, publish.
  auto step = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (t + C::NS - 1 < nsteps) issue(qt0 + t + C::NS - 1, (buf + C::NS - 1) % C::NS);
    const int qs0 = (qt0 + t) * C::BQ;
    const uint32_t* Bb = Bs[DROP ? buf : 0];
    if (qs0 < k0 + C::BN)
      dkdv_step_diag<E, HS, DROP, KVL>(Qs[buf], Gs[buf], Ls[buf], Ds[buf], Bb, KVs, krow - k0, qs0, kw0,
                                  krow, h, c, L, R, gl);
    else
      dkdv_step_full<E, HS, DROP, KVL>(Qs[buf], Gs[buf], Ls[buf], Ds[buf], Bb, KVs, krow - k0, qs0,
                                  krow, h, c, L, R, gl);
    wait_ring<C::NS, PER>(max(0, min(C::NS - 2, nsteps - t - 2)));
    if constexpr (DsOf<E>::kConvert)
      if (t + 1 < nsteps) dma_tile_to_f16<HS, C::BQ, C::NW>(Qs[(buf + 1) % C::NS], w, lane);
    __syncthreads();
  };
  ring_loop<C::NS>(nsteps, step);

  // dK^T / dV^T register i of lane (n, h): column d = db*32 + 8*(i/4) + 4h + i%4, key krow.
  const int64_t gbase = slice_base<HS, STRIDED>(lg, bh, H, T);
  const uint32_t gbytes = slice_bytes_of<HS, STRIDED>(lg, T);
  const rsrc_t wk = make_rsrc(dk + gbase, gbytes), wv = make_rsrc(dv + gbase, gbytes);
  const int rsg = STRIDED ? int(lg.st) : HS;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = uint32_t(krow * rsg + db * 32 + 8 * g + 4 * h) * 2;
      bstore8(wv, off, u32x2{E::pack(R.dva[db][4 * g], R.dva[db][4 * g + 1]),
                             E::pack(R.dva[db][4 * g + 2], R.dva[db][4 * g + 3])});
      bstore8(wk, off, u32x2{E::pack(R.dka[db][4 * g] * scale, R.dka[db][4 * g + 1] * scale),
                             E::pack(R.dka[db][4 * g + 2] * scale, R.dka[db][4 * g + 3] * scale)});
    }
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 4 wavefronts = 128 queries of one (b, h); wavefront w keeps
// queries r0 + 32w .. +31 (Q^T and dO^T as MFMA B operands, lse and D as
// per-lane scalars) and the dQ^T accumulator in registers.  Steps walk 64-key
// tiles from 0 to the diagonal.  Per step and 32-key block:
//   S^T = K Q^T, dP^T = V dO^T      C[key][query]; K, V rows from LDS in
//                                   perm_row order (8 consecutive keys per
//                                   lane in registers 8t..8t+7)
//   dS^T (f32) -> fp16               the B operand of
//   dQ^T += K^T dS^T                 C[d][query]; K^T via LDS transpose reads
// The walk starts from the row term D~ = rowsum(dO * O) of the stored 16-bit
// O, which is off by up to half an ulp of each O element.  The exact row term
// is D = sum_j P dP (sum_j P = 1), so with dS~ = P (dP - D~):
//   eps = D - D~ = sum_j dS~,   dQ = scale (sum_j dS~ K - eps sum_j P K),
// i.e. the kernel also accumulates M^T += K^T P^T (same K^T operands) and the
// float32 row sums of dS~, and writes the exact D to the workspace for the
// dK/dV kernel.  With dropout dS~ = P (Z dP - D~) and the same identities
// hold (sum_j P Z dP = dO . O).  The keep decisions either are drawn here
// and each byte (query, 8-key group) is stored for the dK/dV kernel
// (DROP == kDropDraw; layout there), or come from the bytes the forward
// stored (kDropRead), DMA'd into LDS step by step like the K and V tiles.
// K and Q^T are fp16 (see DsOf): the K tile is converted in place as it
// lands, Q^T once.
// Dropout modes of the dQ kernel.
enum DqDrop { kDropNone = 0, kDropDraw = 1, kDropRead = 2 };

template <int HS>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int BM = 32 * NW;  // queries per workgroup
  static constexpr int BN = 64;       // keys per step
  static constexpr int KSTEP = HS / 16;
  static constexpr int DB = HS / 32;
  static constexpr int NS = 3;  // LDS ring depth: tile t computes while t+1 converts and t+2 lands
  static constexpr int PER = 2 * (BN * HS / 512) / NW;  // DMA instructions per wavefront per step
  static constexpr int KEEP_WORDS = (BM / 8) * (BN / 8) * 2;  // keep-bit tile (kDropRead), words
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

// `between` runs once the first block's S and dP MFMAs are issued (the ring's
// DMA issue and tile conversion, which then overlap the matrix core's work).
// Bb (kDropRead): the step's keep-bit tile; kbo: this lane's byte offset in
// it for key group 0 (query octet and byte of qrow); h: lane half.
template <class E, int HS, int KIND, int DROP, class F>
__device__ __forceinline__ void dq_step(const uint16_t* Kb, const uint16_t* Vb, int dn, float c,
                                        float lse2, float Dq, const LaneOffsets<HS>& L,
                                        const u32x4 (&qf)[HS / 16], const u32x4 (&gf)[HS / 16],
                                        f32x16 (&dqa)[HS / 32], f32x16 (&mka)[HS / 32],
                                        float& esum, const f32x16& negD, uint32_t qrow,
                                        uint32_t g0, uint32_t bh, const Dropout& dr,
                                        rsrc_t rb, uint32_t ng, const uint8_t* Bb, int kbo,
                                        int h, F&& between) {
  using C = DqCfg<HS>;
  using Ed = typename DsOf<E>::T;
  constexpr int NKB = KIND == kDiagLo ? 1 : 2;  // 32-key blocks computed
  constexpr int KD = KIND == kDiagLo ? 0 : (KIND == kDiagHi ? 1 : -1);  // the diagonal block
  u32x4 dsp[2][2], pp[2][2];
  // Keep bits of the step's runs, drawn (and stored) before the S / dP MFMAs
  // so that the generator's vector ALU work overlaps them, or read.
  uint32_t bits[2][2] = {{0xFFu, 0xFFu}, {0xFFu, 0xFFu}};
  if constexpr (DROP == kDropDraw) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t G = g0 + 4 * kb + 2 * t;
        bits[kb][t] = keep_bits8(qrow, G, bh, dr);
        if (G < ng) bstore1(rb, ((qrow >> 3) * ng + G) * 8 + (qrow & 7), bits[kb][t]);
      }
  } else if constexpr (DROP == kDropRead) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) bits[kb][t] = Bb[kbo + 8 * (4 * kb + 2 * t + h)];
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    // The dP accumulator starts from -D~ (every register of a lane is this
    // lane's query; with dropout -D~/zs), so it ends as dP - D~ (dP - D~/zs).
    f32x16 st = {}, dpt = negD;
#pragma unroll
    for (int ks = 0; ks < C::KSTEP; ++ks) {
      st = Ed::mfma(op_nat<HS>(Kb, L, kb * 32, ks), qf[ks], st);
      dpt = E::mfma(op_nat<HS>(Vb, L, kb * 32, ks), gf[ks], dpt);
    }
    if (kb == 0) {
      __builtin_amdgcn_sched_barrier(0);
      between();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float pv[8], dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float p = __builtin_amdgcn_exp2f(fmaf(st[8 * t + e], c, -lse2));
        if (kb == KD && 16 * t + e > dn) p = 0.f;
        pv[e] = p;
        if constexpr (DROP) {  // p is P zs here, Dq is D~ / zs
          const uint32_t m = keep_mask(bits[kb][t], e);
          dsv[e] = p * __uint_as_float((__float_as_uint(dpt[8 * t + e]) & m) |
                                       (__float_as_uint(-Dq) & ~m));
        } else {
          dsv[e] = p * dpt[8 * t + e];
        }
        esum += dsv[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsp[kb][t][e] = Ed::pack(dsv[2 * e], dsv[2 * e + 1]);
        pp[kb][t][e] = Ed::pack(pv[2 * e], pv[2 * e + 1]);

      }
    }
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const u32x4 kt = op_tr<HS>(Kb, L, kb * 32 + 16 * t, db);
        dqa[db] = Ed::mfma(kt, dsp[kb][t], dqa[db]);
        mka[db] = Ed::mfma(kt, pp[kb][t], mka[db]);
      }
}

template <class E, int HS, bool STRIDED, int DROP>  // STRIDED as for the dK/dV kernel; DqDrop
__global__ __launch_bounds__(kThreads, DROP ? GATTN_DQ_DROP_OCC : GATTN_DQ_OCC) void dq16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, float* __restrict__ Dg,
    float* __restrict__ L2g, uint64_t* __restrict__ keep, uint16_t* __restrict__ dq, int BH,
    int H, int T, float scale, Layout li, Layout lo, Layout lg, Dropout dr) {
  using C = DqCfg<HS>;
  constexpr bool READ = DROP == kDropRead;
  constexpr int PER = C::PER + (READ ? 1 : 0);
  __shared__ __attribute__((aligned(16))) uint16_t Ks[C::NS][C::BN * HS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[C::NS][C::BN * HS];
  __shared__ __attribute__((aligned(16))) uint32_t Bs[READ ? C::NS : 1][READ ? C::KEEP_WORDS : 4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int nqt = (T + C::BM - 1) / C::BM;
  const int BH8 = heads_padded(BH);
  const int qt = nqt - 1 - int(blockIdx.x) / BH8;  // heaviest query tiles first
  const int bh = int(blockIdx.x) % BH8;
  if (bh >= BH) return;  // grid padding (uniform in the workgroup, before any barrier)
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
  // Keep bytes (DROP): this slice's ng x ng blocks of 8 bytes.  kbo: this
  // lane's byte in the step's keep-bit tile (16 query octets x 8 key groups
  // of 8 bytes) for key group 0.
  const uint32_t ng = uint32_t(T + 7) >> 3;
  const rsrc_t rb = make_rsrc(DROP ? keep + int64_t(bh) * ng * ng : keep, ng * ng * 8);
  const int kbo = ((qrow - r0) >> 3) * 64 + (qrow & 7);

  auto issue = [&](int kt, int buf) {
    dma_tile<HS, C::BN, C::NW>(rk, kt * C::BN, rs, Ks[buf], w, lane);
    dma_tile<HS, C::BN, C::NW>(rv, kt * C::BN, rs, Vs[buf], w, lane);
    if constexpr (READ) {
      // Wavefront w: query octets 4w .. 4w+3 of the workgroup, the step's 8
      // key groups each (lane: octet 4w + lane/4, groups 2 (lane%4) and +1).
      constexpr int KQ = C::KEEP_WORDS / C::NW;  // words per wavefront
      const uint32_t qo = uint32_t(r0 / 8 + 4 * w + (lane >> 2));
      if (lane < 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(Bs[buf] + w * KQ), 16,
            (qo * ng + uint32_t(kt * (C::BN / 8)) + 2u * uint32_t(lane & 3)) * 8, 0, 0, 0);
    }
  };
  const int nkt = (min(r0 + C::BM, T) - 1) / C::BN + 1;
  issue(0, 0);

  // Q^T, dO^T fragments (lane (n, h): row qrow, columns 16 ks + 8h .. +7), and
  // D~ = rowsum(dO * O) of this lane's query from the same columns of O.
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
  const float lse2 = bloadf(make_rsrc(lse + long(bh) * T, uint32_t(T) * 4), uint32_t(qrow) * 4) *
                     kLog2e;
  if (1 < nkt) issue(1, 1);
  // With dropout the weights come out as P zs and the row term as D~ / zs.
  const float Dq = DROP ? halves_sum(dpart) * dr.izs : halves_sum(dpart);
  const float lse2x = DROP ? lse2 - dr.lzs : lse2;
  if constexpr (DsOf<E>::kConvert) {
#pragma unroll
    for (int ks = 0; ks < C::KSTEP; ++ks) qf[ks] = bf16x8_to_f16x8(qf[ks]);
  }
  f32x16 dqa[C::DB], mka[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dqa[db] = mka[db] = f32x16{};
  float esum = 0.f;
  f32x16 negD;
#pragma unroll
  for (int i = 0; i < 16; ++i) negD[i] = -Dq;

  const LaneOffsets<HS> L(lane);
  // Tile 0 and this wavefront's q, dO, O, lse rows (tile 1's DMA, issued
  // last, may still be in flight).
  if (1 < nkt)
    wait_vmem_n<PER>();
  else
    wait_vmem();
  if constexpr (DsOf<E>::kConvert) dma_tile_to_f16<HS, C::BN, C::NW>(Ks[0], w, lane);
  __syncthreads();
  // One step, tile kt in buffer kt % 3 (landed, converted and published by
  // the previous barrier): wait for this wavefront's DMA of tile kt+1 (the
  // only one in flight), then, once the first S / dP MFMAs are issued, start
  // the DMA of tile kt+2 into the buffer tile kt-1 left (every wavefront
  // passed the previous barrier after reading it) and convert this
  // wavefront's part of tile kt+1; compute tile kt; publish.
  auto step = [&](int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    wait_vmem();
    auto between = [&] {
      if (kt + 2 < nkt) issue(kt + 2, (buf + 2) % C::NS);
      if constexpr (DsOf<E>::kConvert)
        if (kt + 1 < nkt) dma_tile_to_f16<HS, C::BN, C::NW>(Ks[(buf + 1) % C::NS], w, lane);
    };
    const int key0 = kt * C::BN;
    const uint32_t g0 = uint32_t(key0 / 8 + h), ub = uint32_t(bh), uq = uint32_t(qrow);
    if (q0 < T && key0 <= q0) {
      if (key0 == q0)
        dq_step<E, HS, kDiagLo, DROP>(Ks[buf], Vs[buf], dn, c, lse2x, Dq, L, qf, gf, dqa, mka, esum,
                                      negD, uq, g0, ub, dr, rb, ng,
                                      reinterpret_cast<const uint8_t*>(Bs[READ ? buf : 0]), kbo, h,
                                      between);
      else if (key0 + 32 == q0)
        dq_step<E, HS, kDiagHi, DROP>(Ks[buf], Vs[buf], dn, c, lse2x, Dq, L, qf, gf, dqa, mka, esum,
                                      negD, uq, g0, ub, dr, rb, ng,
                                      reinterpret_cast<const uint8_t*>(Bs[READ ? buf : 0]), kbo, h,
                                      between);
      else
        dq_step<E, HS, kFull, DROP>(Ks[buf], Vs[buf], dn, c, lse2x, Dq, L, qf, gf, dqa, mka, esum,
                                    negD, uq, g0, ub, dr, rb, ng,
                                      reinterpret_cast<const uint8_t*>(Bs[READ ? buf : 0]), kbo, h,
                                      between);
    } else {
      between();
    }
    __syncthreads();
  };
  ring_loop<C::NS>(nkt, step);

  // eps = D - D~ (both halves of the wavefront hold this query's keys).
  // dQ^T register i of lane (n, h): column d = db*32 + 8*(i/4) + 4h + i%4, query qrow.
  // With dropout: eps as without (sum_j P (Z dP - D~)), Dq = D~/zs, M summed
  // from P zs, and the workspace takes D/zs and L2 - log2 zs.
  const float eps = halves_sum(esum);
  const float epm = DROP ? eps * dr.izs : eps;  // eps against the M accumulator
  if (h == 0) {
    bstoref(make_rsrc(Dg + long(bh) * T, uint32_t(T) * 4), uint32_t(qrow) * 4, Dq + epm);
    bstoref(make_rsrc(L2g + long(bh) * T, uint32_t(T) * 4), uint32_t(qrow) * 4, lse2x);
  }
  const rsrc_t wq = make_rsrc(dq + slice_base<HS, STRIDED>(lg, bh, H, T),
                              slice_bytes_of<HS, STRIDED>(lg, T));
  const int rsg = STRIDED ? int(lg.st) : HS;
  auto fin = [&](int db, int i) { return fmaf(-epm, mka[db][i], dqa[db][i]) * scale; };
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = uint32_t(qrow * rsg + db * 32 + 8 * g + 4 * h) * 2;
      bstore8(wq, off, u32x2{E::pack(fin(db, 4 * g), fin(db, 4 * g + 1)),
                             E::pack(fin(db, 4 * g + 2), fin(db, 4 * g + 3))});
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
                         const uint16_t* dO, const float* D, const float* L2,
                         const uint64_t* keep, uint16_t* dk, uint16_t* dv, int BH, int H, int T,
                         int hs, float scale, Layout li, Layout lo, Layout lg, const Dropout& dr,
                         hipStream_t s) {
  const int bn = DkdvCfg<64>::BN;
  const dim3 grid(unsigned(((T + bn - 1) / bn) * heads_padded(BH)));
  const bool strided = !all_contiguous(H, T, hs, li, lo, lg);
  auto pick = [&](auto dropc) {
    constexpr bool D = decltype(dropc)::value;
    return hs == 64 ? (strided ? dkdv16_kernel<E, 64, true, D> : dkdv16_kernel<E, 64, false, D>)
                    : (strided ? dkdv16_kernel<E, 32, true, D> : dkdv16_kernel<E, 32, false, D>);
  };
  auto kern = dr.thr != 0 ? pick(std::true_type{}) : pick(std::false_type{});
  return launch(kern, grid, dim3(kThreads), s, q, k, v, dO, D, L2, keep, dk, dv, BH, H, T, scale,
                li, lo, lg, dr);
}

template <class E>
hipError_t dq16_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                       float* L2, uint64_t* keep, bool keep_stored, uint16_t* dq, int BH, int H,
                       int T, int hs, float scale, Layout li, Layout lo, Layout lg,
                       const Dropout& dr, hipStream_t s) {
  const int bm = DqCfg<64>::BM;
  const dim3 grid(unsigned(((T + bm - 1) / bm) * heads_padded(BH)));
  const bool strided = !all_contiguous(H, T, hs, li, lo, lg);
  auto pick = [&](auto dropc) {
    constexpr int D = decltype(dropc)::value;
    return hs == 64 ? (strided ? dq16_kernel<E, 64, true, D> : dq16_kernel<E, 64, false, D>)
                    : (strided ? dq16_kernel<E, 32, true, D> : dq16_kernel<E, 32, false, D>);
  };
  auto kern = dr.thr == 0   ? pick(std::integral_constant<int, kDropNone>{})
              : keep_stored ? pick(std::integral_constant<int, kDropRead>{})
                            : pick(std::integral_constant<int, kDropDraw>{});
  return launch(kern, grid, dim3(kThreads), s, q, k, v, o, dO, lse, D, L2, keep, dq, BH, H, T,
                scale, li, lo, lg, dr);
}
}  // namespace

hipError_t h16_bwd_pre(const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                       float* L2, int BH, int H, int T, int hs, Layout lo, bool f16,
                       hipStream_t s) {
  if (f16) return pre16_launch<F16>(o, dO, lse, D, L2, BH, H, T, hs, lo, s);
  return pre16_launch<Bf16>(o, dO, lse, D, L2, BH, H, T, hs, lo, s);
}

hipError_t h16_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* dO, const float* D, const float* L2,
                        const uint64_t* keep, uint16_t* dk, uint16_t* dv, int BH, int H, int T,
                        int hs, float scale, Layout li, Layout lo, Layout lg, const Dropout& dr,
                        bool f16, hipStream_t s) {
  if (f16)
    return dkdv16_launch<F16>(q, k, v, dO, D, L2, keep, dk, dv, BH, H, T, hs, scale, li, lo, lg,
                              dr, s);
  return dkdv16_launch<Bf16>(q, k, v, dO, D, L2, keep, dk, dv, BH, H, T, hs, scale, li, lo, lg,
                             dr, s);
}

hipError_t h16_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                      float* L2, uint64_t* keep, bool keep_stored, uint16_t* dq, int BH, int H,
                      int T, int hs, float scale, Layout li, Layout lo, Layout lg,
                      const Dropout& dr, bool f16, hipStream_t s) {
  if (f16)
    return dq16_launch<F16>(q, k, v, o, dO, lse, D, L2, keep, keep_stored, dq, BH, H, T, hs, scale,
                            li, lo, lg, dr, s);
  return dq16_launch<Bf16>(q, k, v, o, dO, lse, D, L2, keep, keep_stored, dq, BH, H, T, hs, scale,
                           li, lo, lg, dr, s);
}

}  // namespace gattn
