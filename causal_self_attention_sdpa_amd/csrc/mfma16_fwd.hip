// 16-bit (bf16 or fp16) causal attention forward on gfx950 MFMA
// (v_mfma_f32_32x32x16_bf16 / _f16); E is the element type's traits.
//
// Method ("Let's build GPT" summary page): scores are query.key products of
// earlier tokens (1:06:16) scaled by 1/sqrt(head size) (1:17:18); a
// lower-triangular mask puts -inf above the diagonal (48:54, 55:20); each row
// is softmax-normalised (51:04) and weights the values (1:10:15); heads are
// independent (1:22:27).  The per-row log-sum-exp is written for the backward.
//
// Work split: one workgroup = 4 wavefronts = 128 query rows of one (b, h);
// wavefront w owns rows r0 + 32w .. r0 + 32w + 31.  64-row key and value
// tiles arrive in double-buffered, swizzled LDS tiles by LDS DMA; tiles
// entirely above the diagonal are never loaded, and of the tile on a
// wavefront's diagonal only the 32x32 blocks not entirely above it are
// computed (the mask touches one block).  Per tile and wavefront:
//   S^T (keys x queries) = K Q^T   on MFMA, Q^T held in registers for the
//                                   whole loop (B operand), K rows read from
//                                   LDS in perm_row order so each lane's
//                                   registers 8t..8t+7 are 8 consecutive keys;
//   online softmax in base 2 (reference max m and sum l per query = per
//   lane, so the rescale factor is a per-lane scalar).  A row's reference
//   max m only moves when its weights against the current m would grow past
//   2^8 (the test uses the weights' sums, so the common tile needs no row
//   max), so the weights stay <= 256 (well inside the 16-bit and float32
//   ranges) and the output is rescaled only on those rare halves;
//   O^T (hs x queries) += V^T P^T  on MFMA, P^T straight from the S^T
//                                   accumulators (no LDS round trip), V^T
//                                   read from the row-major V tile with LDS
//                                   transpose reads.
// With dropout (DROP), each weight's keep decision comes from the counter-
// based generator of philox.h: the lane's run of 8 consecutive keys of one
// query is exactly one generator block.  The row sum l takes the weights
// before dropout (the softmax is normalised first), the value sum only the
// kept ones, and the output is multiplied by 1/(1 - p) with 1/l.  If the
// caller gives a keep buffer, each run's 8 decisions are also stored there as
// one byte of the 8x8 keep-bit blocks the backward kernels read (block (query
// octet I, key group G) at bytes (I * ng + G) * 8 of the slice's part, byte e
// = query 8I + e, bit r = key 8G + r, ng = ceil(T / 8)).
// Tensors are addressed through Layout strides (q, k, v: li; o: lo), so the
// fused (B, T, 3C) projection output and a (B, T, C) output are read and
// written in place.  Rows past T are read as zeros (buffer resources sized to
// the span of one (b, h) slice); keys past T are always above the diagonal of
// every real query, so the mask removes them, and stores of rows past T are
// dropped.
#include <cmath>

#include "mfma16_common.h"
#include "gattn_internal.h"
#include "philox.h"

#ifndef GATTN_FWD_STAGES
#define GATTN_FWD_STAGES 2
#endif

namespace gattn {
namespace {

constexpr int kThreads = 256;

template <int HS>
struct FwdCfg {
  static constexpr int NW = 4;            // wavefronts per workgroup
  static constexpr int BM = 32 * NW;      // query rows per workgroup
  static constexpr int BN = 64;           // key rows per tile
  static constexpr int KSTEP = HS / 16;   // MFMA k-steps over hs
  static constexpr int DB = HS / 32;      // 32-wide blocks of hs
  static constexpr int NS = GATTN_FWD_STAGES;            // LDS ring depth
  static constexpr int PER = 2 * (BN * HS / 512) / NW;  // DMA instructions per wavefront per tile
  static_assert((BN * HS / 512) % NW == 0, "uniform DMA split");
};

template <int HS>
struct FwdState {
  f32x16 oacc[HS / 32];
  float m, l;
};

// Kinds of key tile for one wavefront (32 queries q0 .. q0+31, 64 keys from
// key0, q0 - key0 a multiple of 32):
//   kFull  : every key <= every query;
//   kDiagLo: key0 == q0, so keys key0 .. key0+31 form the 32x32 diagonal
//            block and keys key0+32 .. key0+63 lie above every query (skipped);
//   kDiagHi: key0 + 32 == q0: the first 32 keys are full, the second 32 form
//            the diagonal block.
enum TileKind { kFull = 0, kDiagLo = 1, kDiagHi = 2 };

// The weights of one 32-key half (registers s of a score block) against the
// reference max m (mc = m * c): P^T operand pairs in pf and, returned, the
// lane's sum of its 16 weights before dropout.  bits: the two 8-key runs'
// keep bits (DROP).
template <class E, bool DROP>
__device__ __forceinline__ float half_weights(const f32x16& s, float c, float mc,
                                              const uint32_t (&bits)[2], u32x4 (&pf)[2]) {
  float ls;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * t + 2 * e], c, -mc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * t + 2 * e + 1], c, -mc));
      if constexpr (DROP)
        pf[t][e] = E::pack(keep_or_zero(p0, bits[t], 2 * e), keep_or_zero(p1, bits[t], 2 * e + 1));
      else
        pf[t][e] = E::pack(p0, p1);
      ls = t == 0 && e == 0 ? p0 + p1 : ls + (p0 + p1);
    }
  return ls;
}

// One key tile for one wavefront.  `dn` = n - 8h: in the diagonal block,
// register i of lane (n, h) holds key (q0 + 16*(i/8) + 8h + i%8), which lies
// above query q0 + n exactly when 16*(i/8) + i%8 > dn.  With DROP, the run of
// registers 8t..8t+7 of half kh is keys 8 * (g0 + 4 kh + 2 t) .. +7 of query
// qrow (g0 = key0 / 8 + h).
//
// The tile's weights are first formed against the row's current reference
// max m; only a row whose weights in one of its two lanes sum past 2^8, or
// are not finite (the row's first tile, where m = -inf, or a NaN or infinite
// score), moves m to its running maximum, rescales l and O and forms the
// tile's weights again.
// So every weight that reaches the MFMA or l is <= 2^8 (well inside the 16-bit
// and float32 ranges), the row max is computed only on those rare tiles, and
// the decision is per row: a row's result never depends on other rows.
template <class E, int HS, int KIND, bool DROP>
__device__ __forceinline__ void fwd_tile(const uint16_t* Kb, const uint16_t* Vb, int n, int dn,
                                         float c, const LaneOffsets<HS>& L,
                                         const u32x4 (&qf)[HS / 16], FwdState<HS>& st,
                                         uint32_t qrow, uint32_t g0, uint32_t bh,
                                         const Dropout& dr, bool store, rsrc_t rb, uint32_t ng) {
  using C = FwdCfg<HS>;
  constexpr int NKH = KIND == kDiagLo ? 1 : 2;  // 32-key halves computed
  // Keep bits, drawn (and stored) before the S MFMAs: the generator's vector
  // ALU work overlaps them, and the stores have the tile to complete.
  uint32_t bits[2][2] = {{0xFFu, 0xFFu}, {0xFFu, 0xFFu}};
  if constexpr (DROP) {
#pragma unroll
    for (int kh = 0; kh < NKH; ++kh)
#pragma unroll
      for (int t = 0; t < 2; ++t) bits[kh][t] = keep_bits8(qrow, g0 + 4 * kh + 2 * t, bh, dr);
    if (store)
#pragma unroll
      for (int kh = 0; kh < NKH; ++kh)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t G = g0 + 4 * kh + 2 * t;
          if (G < ng) bstore1(rb, ((qrow >> 3) * ng + G) * 8 + (qrow & 7), bits[kh][t]);
        }
  }
  f32x16 s[2];
#pragma unroll
  for (int kh = 0; kh < NKH; ++kh) {
    s[kh] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KSTEP; ++ks)
      s[kh] = E::mfma(op_nat<HS>(Kb, L, kh * 32, ks), qf[ks], s[kh]);
  }
  // Register i of s[kh] is key key0 + kh*32 + 16*(i/8) + 8h + i%8, query q0 + n.
  if (KIND != kFull) {
    constexpr int kd = KIND == kDiagLo ? 0 : 1;  // the diagonal half
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (16 * (i >> 3) + (i & 7) > dn) s[kd][i] = -INFINITY;
  }
  u32x4 pf[2][2];
  float ls = half_weights<E, DROP>(s[0], c, st.m * c, bits[0], pf[0]);
  if constexpr (NKH == 2) ls += half_weights<E, DROP>(s[1], c, st.m * c, bits[1], pf[1]);
  const uint64_t over = __builtin_amdgcn_ballot_w64(!(ls <= 256.f));
  if (over) {
    const uint32_t rows = uint32_t(over) | uint32_t(over >> 32);
    float mh = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kh = 0; kh < NKH; ++kh)
#pragma unroll
      for (int i = kh == 0 ? 2 : 0; i < 16; i += 2) mh = fmaxf(fmaxf(mh, s[kh][i]), s[kh][i + 1]);
    mh = halves_max(mh);
    // Rows that keep m are multiplied by exactly 1; m = -inf gives alpha = 0.
    const float mn = (rows >> n) & 1u ? fmaxf(st.m, mh) : st.m;
    const float alpha = __builtin_amdgcn_exp2f((st.m - mn) * c);
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) st.oacc[db] *= alpha;
    st.m = mn;
    ls = half_weights<E, DROP>(s[0], c, st.m * c, bits[0], pf[0]);
    if constexpr (NKH == 2) ls += half_weights<E, DROP>(s[1], c, st.m * c, bits[1], pf[1]);
  }
  st.l += ls;
#pragma unroll
  for (int kh = 0; kh < NKH; ++kh)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        st.oacc[db] = E::mfma(op_tr<HS>(Vb, L, kh * 32 + 16 * t, db), pf[kh][t], st.oacc[db]);
}

// STRIDED = false: q, k, v and o are contiguous (B, H, T, hs) and the row
// strides are the compile-time HS.  DROP: dropout with the parameters dr.
template <class E, int HS, bool STRIDED, bool DROP>
__global__ __launch_bounds__(kThreads) void fwd16_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           uint16_t* __restrict__ o,
                                                           float* __restrict__ lse,
                                                           uint64_t* __restrict__ keep, int BH,
                                                           int H, int T, float scale, Layout li,
                                                           Layout lo, Dropout dr) {
  using C = FwdCfg<HS>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[C::NS][C::BN * HS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[C::NS][C::BN * HS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int nqt = (T + C::BM - 1) / C::BM;
  // Heaviest query tiles (most key tiles under the diagonal) first.
  const int BH8 = heads_padded(BH);
  const int qt = nqt - 1 - int(blockIdx.x) / BH8;
  const int bh = int(blockIdx.x) % BH8;
  if (bh >= BH) return;  // grid padding (uniform in the workgroup, before any barrier)
  const int64_t base = slice_base<HS, STRIDED>(li, bh, H, T);
  const uint32_t slice_bytes = slice_bytes_of<HS, STRIDED>(li, T);
  const int rs = STRIDED ? int(li.st) : HS;
  const rsrc_t rq = make_rsrc(q + base, slice_bytes), rk = make_rsrc(k + base, slice_bytes);
  const rsrc_t rv = make_rsrc(v + base, slice_bytes);

  const int r0 = qt * C::BM;
  const int q0 = r0 + 32 * w;  // first query row of this wavefront
  const int qrow = q0 + n;
  const int nkt = (min(r0 + C::BM, T) - 1) / C::BN + 1;
  const float c = scale * kLog2e;
  // Keep bytes (DROP with a keep buffer): this slice's ng x ng blocks.
  const uint32_t ng = uint32_t(T + 7) >> 3;
  const bool store = DROP && keep != nullptr;
  const rsrc_t rb = make_rsrc(store ? keep + int64_t(bh) * ng * ng : keep, store ? ng * ng * 8 : 0);

  auto issue = [&](int kt, int buf) {
    dma_tile<HS, C::BN, C::NW>(rk, kt * C::BN, rs, Ks[buf], w, lane);
    dma_tile<HS, C::BN, C::NW>(rv, kt * C::BN, rs, Vs[buf], w, lane);
  };
#pragma unroll
  for (int j = 0; j < C::NS - 1; ++j)
    if (j < nkt) issue(j, j);

  // Q^T as the MFMA B operand: lane (n, h) holds Q[qrow][16 ks + 8h .. +7].
  u32x4 qf[C::KSTEP];
#pragma unroll
  for (int ks = 0; ks < C::KSTEP; ++ks)
    qf[ks] = bload16(rq, uint32_t(qrow * rs + 16 * ks + 8 * h) * 2);

  FwdState<HS> st;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) st.oacc[db] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const int dn = n - 8 * h;
  const LaneOffsets<HS> L(lane);

  wait_vmem();
  __syncthreads();
  // One tile: prefetch tile kt+NS-1 into the buffer freed by tile kt-1,
  // compute tile kt, wait until tile kt+1 has landed, publish.
  auto step = [&](int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (kt + C::NS - 1 < nkt) issue(kt + C::NS - 1, (buf + C::NS - 1) % C::NS);
    const int key0 = kt * C::BN;
    const uint32_t g0 = uint32_t(key0 / 8 + h);
    if (q0 < T && key0 <= q0) {  // this wavefront sees some key of the tile
      if (key0 == q0)
        fwd_tile<E, HS, kDiagLo, DROP>(Ks[buf], Vs[buf], n, dn, c, L, qf, st, qrow, g0, bh, dr,
                                         store, rb, ng);
      else if (key0 + 32 == q0)
        fwd_tile<E, HS, kDiagHi, DROP>(Ks[buf], Vs[buf], n, dn, c, L, qf, st, qrow, g0, bh, dr,
                                         store, rb, ng);
      else
        fwd_tile<E, HS, kFull, DROP>(Ks[buf], Vs[buf], n, dn, c, L, qf, st, qrow, g0, bh, dr,
                                         store, rb, ng);
    }
    wait_ring<C::NS, C::PER>(max(0, min(C::NS - 2, nkt - kt - 2)));
    __syncthreads();
  };
  ring_loop<C::NS>(nkt, step);

  // The first processed tile holds key 0 <= every query, so m is finite and
  // l > 0 for every real row.  O^T register i of lane (n, h): column
  // d = db*32 + 8*(i/4) + 4h + i%4 of row qrow.
  const float lt = halves_sum(st.l);
  const float inv = (DROP ? dr.zs : 1.f) / lt;
  const rsrc_t wo = make_rsrc(o + slice_base<HS, STRIDED>(lo, bh, H, T),
                              slice_bytes_of<HS, STRIDED>(lo, T));
  const int rso = STRIDED ? int(lo.st) : HS;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = uint32_t(qrow * rso + db * 32 + 8 * g + 4 * h) * 2;
      bstore8(wo, off, u32x2{E::pack(st.oacc[db][4 * g] * inv, st.oacc[db][4 * g + 1] * inv),
                             E::pack(st.oacc[db][4 * g + 2] * inv, st.oacc[db][4 * g + 3] * inv)});
    }
  if (lse != nullptr && h == 0)
    bstoref(make_rsrc(lse + long(bh) * T, uint32_t(T) * 4), uint32_t(qrow) * 4,
            st.m * scale + logf(lt));
}

}  // namespace

namespace {
template <class E>
hipError_t fwd16_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                        float* lse, uint64_t* keep, int BH, int H, int T, int hs, float scale,
                        Layout li, Layout lo, const Dropout& dr, hipStream_t s) {
  const int bm = FwdCfg<64>::BM;
  const dim3 grid(unsigned(((T + bm - 1) / bm) * heads_padded(BH)));
  const bool strided = !all_contiguous(H, T, hs, li, lo, lo);
  auto pick = [&](auto dropc) {
    constexpr bool D = decltype(dropc)::value;
    return hs == 64 ? (strided ? fwd16_kernel<E, 64, true, D> : fwd16_kernel<E, 64, false, D>)
                    : (strided ? fwd16_kernel<E, 32, true, D> : fwd16_kernel<E, 32, false, D>);
  };
  auto kern = dr.thr != 0 ? pick(std::true_type{}) : pick(std::false_type{});
  return launch(kern, grid, dim3(kThreads), s, q, k, v, o, lse, dr.thr != 0 ? keep : nullptr, BH,
                H, T, scale, li, lo, dr);
}
}  // namespace

hipError_t h16_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                   float* lse, uint64_t* keep, int BH, int H, int T, int hs, float scale,
                   Layout li, Layout lo, const Dropout& dr, bool f16, hipStream_t s) {
  if (f16) return fwd16_launch<F16>(q, k, v, o, lse, keep, BH, H, T, hs, scale, li, lo, dr, s);
  return fwd16_launch<Bf16>(q, k, v, o, lse, keep, BH, H, T, hs, scale, li, lo, dr, s);
}

}  // namespace gattn
