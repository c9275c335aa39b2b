// bf16 causal attention forward on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Method ("Let's build GPT" summary page): scores are query.key products of
// earlier tokens (1:06:16) scaled by 1/sqrt(head size) (1:17:18); a
// lower-triangular mask puts -inf above the diagonal (48:54, 55:20); each row
// is softmax-normalised (51:04) and weights the values (1:10:15); heads are
// independent (1:22:27).  The per-row log-sum-exp is written for the backward.
//
// Work split: one workgroup = 4 wavefronts = 128 query rows of one (b, h);
// wavefront w owns rows r0 + 32w .. r0 + 32w + 31.  Key/value tiles of 64
// rows stream through LDS; tiles entirely above the diagonal are never loaded.
// Per tile and wavefront:
//   S^T (keys x queries) = K Q^T   on MFMA, Q^T held in registers for the
//                                   whole loop (B operand), K read from LDS;
//   online softmax in base 2 (running max m, running sum l, per query =
//   per lane, so the rescale factor is a per-lane scalar);
//   O^T (hs x queries) += V^T P^T  on MFMA, P^T straight from the S^T
//                                   accumulators (no LDS round trip), V^T
//                                   read from LDS.
// K rows are fed to the MFMA A operand in a permuted order (bits 2 and 3 of
// the row index swapped) so that each lane's 8 consecutive accumulator
// registers hold 8 consecutive keys: exactly the B-operand layout of the
// second MFMA.  V is transposed on its way into LDS (register pair swizzle),
// so both MFMAs read 16-byte LDS vectors.  Global loads for tile t+1 are
// issued before tile t is computed.
#include <cmath>

#include "bf16_common.h"
#include "gattn_internal.h"

namespace gattn {
namespace {

template <int HS>
struct FwdCfg {
  static constexpr int NW = 4;              // wavefronts per workgroup
  static constexpr int BM = 32 * NW;        // query rows per workgroup
  static constexpr int BN = 64;             // key rows per tile
  static constexpr int KST = HS + 8;        // LDS row stride of K (elements)
  static constexpr int VST = BN + 8;        // LDS row stride of V^T (elements)
  static constexpr int KSTEP = HS / 16;     // MFMA k-steps over hs
  static constexpr int DB = HS / 32;        // 32-wide blocks of hs
  static constexpr int KPT = BN * HS / 8 / (64 * NW);  // 16-byte K chunks per thread
  static constexpr int VU = (BN / 8) * (HS / 2);        // V transpose units (8 keys x 2 d)
  static_assert(KPT >= 1 && VU % 64 == 0 && VU <= 64 * NW, "tile shape");
};

template <int HS>
__global__ __launch_bounds__(256) void bf16_fwd_kernel(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v,
                                                      uint16_t* __restrict__ o,
                                                      float* __restrict__ lse, int BH, int T,
                                                      float scale) {
  using C = FwdCfg<HS>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[C::BN * C::KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[HS * C::VST];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int nqt = (T + C::BM - 1) / C::BM;
  // Heaviest query tiles (most key tiles under the diagonal) first.
  const int qt = nqt - 1 - int(blockIdx.x) / BH;
  const int bh = int(blockIdx.x) % BH;
  const long base = long(bh) * T * HS;
  const uint16_t* qb = q + base;
  const uint16_t* kb = k + base;
  const uint16_t* vb = v + base;

  const int r0 = qt * C::BM;
  const int q0 = r0 + 32 * w;  // first query row of this wavefront
  const int nkt = (min(r0 + C::BM, T) - 1) / C::BN + 1;
  const float c = scale * kLog2e;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // Q^T as the MFMA B operand: lane (n, h) holds Q[q0 + n][16 ks + 8h .. +7].
  const int qrow = q0 + n;
  u32x4 qf[C::KSTEP];
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks)
    qf[ks] = qrow < T ? *reinterpret_cast<const u32x4*>(qb + long(qrow) * HS + 16 * ks + 8 * h)
                      : zero4;

  // Register staging of the next K / V tile.
  u32x4 kr[C::KPT];
  uint32_t vr[8];
  auto gload = [&](int kt) {
    const int key0 = kt * C::BN;
#pragma unroll
    for (int j = 0; j < C::KPT; ++j) {
      const int ch = tid + 256 * j, row = ch / (HS / 8), col = ch % (HS / 8);
      const int key = key0 + row;
      kr[j] = key < T ? *reinterpret_cast<const u32x4*>(kb + long(key) * HS + col * 8) : zero4;
    }
    if (tid < C::VU) {
      const int dp = tid % (HS / 2), kg = tid / (HS / 2);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int key = key0 + kg * 8 + r;
        vr[r] = key < T ? *reinterpret_cast<const uint32_t*>(vb + long(key) * HS + 2 * dp) : 0u;
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < C::KPT; ++j) {
      const int ch = tid + 256 * j, row = ch / (HS / 8), col = ch % (HS / 8);
      *reinterpret_cast<u32x4*>(Ks + row * C::KST + col * 8) = kr[j];
    }
    if (tid < C::VU) {
      const int dp = tid % (HS / 2), kg = tid / (HS / 2);
      u32x4 lo, hi;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lo[t] = (vr[2 * t] & 0xffffu) | (vr[2 * t + 1] << 16);
        hi[t] = (vr[2 * t] >> 16) | (vr[2 * t + 1] & 0xffff0000u);
      }
      *reinterpret_cast<u32x4*>(Vt + (2 * dp) * C::VST + kg * 8) = lo;
      *reinterpret_cast<u32x4*>(Vt + (2 * dp + 1) * C::VST + kg * 8) = hi;
    }
  };

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int prow = perm_row(n);

  gload(0);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (kt + 1 < nkt) gload(kt + 1);
    const int key0 = kt * C::BN;
    if (q0 >= T || key0 > q0 + 31) continue;  // wavefront has no visible key here

    f32x16 s[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kh][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KSTEP; ++ks) {
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(Ks + (kh * 32 + prow) * C::KST + 16 * ks + 8 * h);
        s[kh] = mfma32(a, qf[ks], s[kh]);
      }
    }
    // Causal mask on tiles that reach past this wavefront's first query.
    if (key0 + C::BN - 1 > q0) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kh * 32 + 16 * (i >> 3) + 8 * h + (i & 7);
          if (key > qrow) s[kh][i] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kh][i]);
    mt = halves_max(mt);
    const float mn = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f((m - mn) * c);
    const float mc = mn * c;
    float ls = 0.f;
    u32x4 pf[2][2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kh][8 * t + 2 * e], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kh][8 * t + 2 * e + 1], c, -mc));
          ls += p0 + p1;
          pf[kh][t][e] = pack_bf16(p0, p1);
        }
    l = l * alpha + ls;
    m = mn;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(Vt + (db * 32 + n) * C::VST + kh * 32 +
                                                          16 * t + 8 * h);
          oacc[db] = mfma32(a, pf[kh][t], oacc[db]);
        }
  }

  if (q0 >= T) return;
  const float lt = halves_sum(l);
  if (qrow < T) {
    const float inv = 1.f / lt;
    uint16_t* orow = o + base + long(qrow) * HS;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 val = {pack_bf16(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                     pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * h) = val;
      }
    if (lse != nullptr && h == 0) lse[long(bh) * T + qrow] = m * scale + logf(lt);
  }
}

}  // namespace

hipError_t bf16_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                    float* lse, int BH, int T, int hs, float scale, hipStream_t s) {
  const int bm = 128;
  const dim3 grid(unsigned(((T + bm - 1) / bm) * BH));
  if (hs == 64)
    return launch(bf16_fwd_kernel<64>, grid, dim3(256), s, q, k, v, o, lse, BH, T, scale);
  return launch(bf16_fwd_kernel<32>, grid, dim3(256), s, q, k, v, o, lse, BH, T, scale);
}

}  // namespace gattn
