// bf16 causal attention backward, main kernel, on gfx950 MFMA.
//
// The pages state only that the model is trained with a backward pass; the
// gradients here are the chain rule of the forward ("Let's build GPT"
// summary page: tril mask 48:54 / 55:20, row softmax 51:04, scaled q.k
// 1:06:16 / 1:17:18, weighted values 1:10:15):
//   P  = exp(scale * Q K^T - lse)        (recomputed, masked above the diagonal)
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D = rowsum(dO * O)
//   dK = scale * dS^T Q,   dQ = scale * dS K.
//
// Work split: one workgroup = 4 wavefronts = 128 keys of one (b, h);
// wavefront w owns keys k0 + 32w .. +31 and keeps them, as MFMA B operands,
// in registers (K and V fragments) for the whole loop, together with its
// dK^T and dV^T accumulators.  The loop walks 64-query tiles from the
// diagonal down (tiles strictly above it are never visited).  Per tile:
//   S  = Q K^T,  dP = dO V^T   (C[query][key]; Q and dO rows from LDS with
//                               the perm_row order, so P and dS land in the
//                               k-slot order of the next MFMAs)
//   P, dS in f32 registers; P = 0 above the diagonal; rows past T carry
//   lse = +inf so their P is exactly 0.
//   dV^T += dO^T P,  dK^T += Q^T dS   (C[d][key]; dO^T and Q^T come from
//                                      the row-major LDS tiles through
//                                      ds_read_b64_tr_b16)
//   dS^T -> LDS; barrier; each wavefront computes one 32x32 block of
//   dQ = dS K (both operands through transpose reads) and adds it to the
//   float32 accumulator in HBM with atomics.
#include <cmath>

#include "bf16_common.h"
#include "gattn_internal.h"

namespace gattn {
namespace {

template <int HS>
struct BwdCfg {
  static constexpr int NW = 4;                  // wavefronts per workgroup
  static constexpr int BN = 32 * NW;            // keys per workgroup
  static constexpr int BQ = 64;                 // queries per loop step
  static constexpr int QB = BQ / 32;            // 32-query blocks per step
  static constexpr int KSTEP = HS / 16;         // MFMA k-steps over hs
  static constexpr int DB = HS / 32;            // 32-wide blocks of hs
  static constexpr int ST = HS + 8;             // LDS row stride of Q, dO, K tiles
  static constexpr int SST = BQ + 8;            // LDS row stride of dS^T
  static constexpr int NBLK = QB * DB;          // 32x32 blocks of a dQ tile
  static constexpr int KSPLIT = NW / NBLK;      // wavefronts sharing one dQ block
  static constexpr int DQ_KSTEPS = BN / 16 / KSPLIT;
  static constexpr int LPT = BQ * HS / 8 / (64 * NW);  // 16-byte chunks per thread per tile
  static_assert(LPT >= 1 && NW % NBLK == 0, "tile shape");
};

template <int HS>
__global__ __launch_bounds__(256) void bf16_bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Dg, float* __restrict__ dq_acc,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int BH, int T, float scale) {
  using C = BwdCfg<HS>;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[C::BQ * C::ST];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[C::BQ * C::ST];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[C::BN * C::ST];
  __shared__ __attribute__((aligned(16))) uint16_t dSt[C::BN * C::SST];
  __shared__ __attribute__((aligned(16))) float lse_s[C::BQ];
  __shared__ __attribute__((aligned(16))) float D_s[C::BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  // Key tiles near the start of the sequence have the most queries below
  // the diagonal: schedule them first.
  const int kt = int(blockIdx.x) / BH;
  const int bh = int(blockIdx.x) % BH;
  const long base = long(bh) * T * HS;
  const int key0 = kt * C::BN;
  const int kw0 = key0 + 32 * w;  // first key of this wavefront
  const float c = scale * kLog2e;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // K, V fragments (B operands of S = Q K^T and dP = dO V^T):
  // lane (n, h) holds row kw0 + n, elements 16 ks + 8h .. +7.
  const int krow = kw0 + n;
  u32x4 kf[C::KSTEP], vf[C::KSTEP];
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks) {
    const long off = base + long(krow) * HS + 16 * ks + 8 * h;
    kf[ks] = krow < T ? *reinterpret_cast<const u32x4*>(k + off) : zero4;
    vf[ks] = krow < T ? *reinterpret_cast<const u32x4*>(v + off) : zero4;
  }
  // Whole K tile, row-major, for the dQ product.
  for (int ch = tid; ch < C::BN * HS / 8; ch += 64 * C::NW) {
    const int row = ch / (HS / 8), col = ch % (HS / 8), key = key0 + row;
    *reinterpret_cast<u32x4*>(Ks + row * C::ST + col * 8) =
        key < T ? *reinterpret_cast<const u32x4*>(k + base + long(key) * HS + col * 8) : zero4;
  }

  f32x16 dka[C::DB], dva[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dka[db][i] = dva[db][i] = 0.f;

  // Register staging of the next query tile.
  u32x4 qr[C::LPT], gr[C::LPT];
  float lr = 0.f, dr = 0.f;
  auto gload = [&](int qt) {
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const int ch = tid + 64 * C::NW * j, row = ch / (HS / 8), col = ch % (HS / 8);
      const int qi = qt * C::BQ + row;
      const long off = base + long(qi) * HS + col * 8;
      qr[j] = qi < T ? *reinterpret_cast<const u32x4*>(q + off) : zero4;
      gr[j] = qi < T ? *reinterpret_cast<const u32x4*>(dO + off) : zero4;
    }
    if (tid < C::BQ) {
      const int qi = qt * C::BQ + tid;
      lr = qi < T ? lse[long(bh) * T + qi] * kLog2e : INFINITY;
      dr = qi < T ? Dg[long(bh) * T + qi] : 0.f;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const int ch = tid + 64 * C::NW * j, row = ch / (HS / 8), col = ch % (HS / 8);
      *reinterpret_cast<u32x4*>(Qs + row * C::ST + col * 8) = qr[j];
      *reinterpret_cast<u32x4*>(dOs + row * C::ST + col * 8) = gr[j];
    }
    if (tid < C::BQ) {
      lse_s[tid] = lr;
      D_s[tid] = dr;
    }
  };

  const int nqt = (T + C::BQ - 1) / C::BQ;
  const int qt0 = key0 / C::BQ;
  const int prow = perm_row(n);
  // dQ block owned by this wavefront in the second phase of each step.
  const int blk = w % C::NBLK, part = w / C::NBLK;
  const int dq_qb = blk / C::DB, dq_db = blk % C::DB;

  gload(qt0);
  for (int qt = qt0; qt < nqt; ++qt) {
    __syncthreads();  // previous step's reads of Qs, dOs, dSt are done
    lstore();
    __syncthreads();
    if (qt + 1 < nqt) gload(qt + 1);
    const int qs0 = qt * C::BQ;

#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KSTEP; ++ks) {
        const int off = (qb * 32 + prow) * C::ST + 16 * ks + 8 * h;
        s = mfma32(*reinterpret_cast<const u32x4*>(Qs + off), kf[ks], s);
        dp = mfma32(*reinterpret_cast<const u32x4*>(dOs + off), vf[ks], dp);
      }
      // Register i of this lane is query qs0 + qb*32 + 16*(i/8) + 8h + i%8, key kw0 + n.
      const bool diag = kw0 + 31 > qs0 + qb * 32;
      u32x4 pp[2], dsp[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ql = qb * 32 + 16 * t + 8 * h;  // local index of the run of 8 queries
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse_s + ql);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse_s + ql + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(D_s + ql);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(D_s + ql + 4);
        float pv[8], dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float le = e < 4 ? l0[e] : l1[e - 4];
          const float De = e < 4 ? d0[e] : d1[e - 4];
          float p = __builtin_amdgcn_exp2f(fmaf(s[8 * t + e], c, -le));
          if (diag && krow > qs0 + ql + e) p = 0.f;
          pv[e] = p;
          dsv[e] = p * (dp[8 * t + e] - De);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pp[t][e] = pack_bf16(pv[2 * e], pv[2 * e + 1]);
          dsp[t][e] = pack_bf16(dsv[2 * e], dsv[2 * e + 1]);
        }
        // dS^T row (this lane's key), queries ql .. ql+7.
        *reinterpret_cast<u32x4*>(dSt + (32 * w + n) * C::SST + ql) = dsp[t];
      }
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int k0 = qb * 32 + 16 * t;
          dva[db] = mfma32(lds_operand_tr(dOs, C::ST, k0, db * 32, lane), pp[t], dva[db]);
          dka[db] = mfma32(lds_operand_tr(Qs, C::ST, k0, db * 32, lane), dsp[t], dka[db]);
        }
    }
    __syncthreads();  // dS^T complete

    // dQ block (queries dq_qb*32 .., hs columns dq_db*32 ..), keys of part `part`.
    f32x16 dqa;
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < C::DQ_KSTEPS; ++kk) {
      const int k0 = (part * C::DQ_KSTEPS + kk) * 16;
      dqa = mfma32(lds_operand_tr(dSt, C::SST, k0, dq_qb * 32, lane),
                   lds_operand_tr(Ks, C::ST, k0, dq_db * 32, lane), dqa);
    }
    // Register i: query qs0 + dq_qb*32 + 8*(i/4) + 4h + i%4, column dq_db*32 + n.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qi = qs0 + dq_qb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
      if (qi < T) unsafeAtomicAdd(dq_acc + base + long(qi) * HS + dq_db * 32 + n, dqa[i] * scale);
    }
  }

  // dK^T, dV^T register i of lane (n, h): column d = db*32 + 8*(i/4) + 4h + i%4, key krow.
  if (krow < T) {
    const long off = base + long(krow) * HS;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * h;
        const u32x2 vv = {pack_bf16(dva[db][4 * g], dva[db][4 * g + 1]),
                          pack_bf16(dva[db][4 * g + 2], dva[db][4 * g + 3])};
        const u32x2 kk = {pack_bf16(dka[db][4 * g] * scale, dka[db][4 * g + 1] * scale),
                          pack_bf16(dka[db][4 * g + 2] * scale, dka[db][4 * g + 3] * scale)};
        *reinterpret_cast<u32x2*>(dv + off + d) = vv;
        *reinterpret_cast<u32x2*>(dk + off + d) = kk;
      }
  }
}

}  // namespace

hipError_t bf16_bwd_main(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, const float* lse, const float* D, float* dq_acc,
                         uint16_t* dk, uint16_t* dv, int BH, int T, int hs, float scale,
                         hipStream_t s) {
  const int bn = 128;
  const dim3 grid(unsigned(((T + bn - 1) / bn) * BH));
  if (hs == 64)
    return launch(bf16_bwd_kernel<64>, grid, dim3(256), s, q, k, v, dO, lse, D, dq_acc, dk, dv,
                  BH, T, scale);
  return launch(bf16_bwd_kernel<32>, grid, dim3(256), s, q, k, v, dO, lse, D, dq_acc, dk, dv, BH,
                T, scale);
}

}  // namespace gattn
