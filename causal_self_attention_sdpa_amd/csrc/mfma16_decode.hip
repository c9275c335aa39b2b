// 16-bit (bf16 or fp16) forward of the newest Tq tokens against Tk >= Tq keys
// on gfx950: decoding with the keys and values of earlier tokens kept.  Tq > 1
// runs the MFMA kernel (dec16_kernel), one new token the vector-ALU kernel
// (dec1_kernel, below); both read every kept key and value once.
//
// Query i is the token at position Tk - Tq + i of the key sequence and sees
// keys j <= Tk - Tq + i: the causal mask of "Let's build GPT" (tril, 48:54;
// -inf fill, 55:20) aligned on the newest token.  The pages' generate
// recomputes the whole forward for every new token (no key/value cache,
// "nanoGPT" notes section 5); the rows computed here are the last Tq rows of
// that forward.
//
// With few queries the work is reading K and V once (HBM-bound), so the key
// range is split twice.  Workgroup (b, h, 32-query block, split s) owns key
// tiles [s*tps, ...) of 64 keys; each of its NW wavefronts streams every
// NW-th of those tiles through its own double-buffered swizzled LDS tiles
// (LDS DMA) and runs the forward's tile step (S^T = K Q^T on MFMA, base-2
// online softmax, O^T += V^T P^T).  The wavefronts then merge their (max,
// sum, output) states through LDS.  With one split the workgroup writes o
// and lse; otherwise it writes its normalised partial output and
// log-sum-exp in float32 and dec16_combine merges the splits:
// lse = log sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s, rounded once
// to the 16-bit type.  Rows (or whole splits) that see no key keep
// m = -inf and l = 0 and contribute exp(-inf) = 0; every step is written so
// that no NaN arises from -inf - (-inf).
#include <cmath>

#include "gattn_internal.h"
#include "mfma16_common.h"

namespace gattn {
namespace {

constexpr int kBN = 64;  // keys per tile

template <int HS>
struct DecState {
  f32x16 oacc[HS / 32];
  float m, l;
};

// One key tile for a 32-query block.  `last` = newest key visible to this
// lane's query; MASK: some key of the tile may lie past it.
template <class E, int HS, bool MASK>
__device__ __forceinline__ void dec_tile(const uint16_t* Kb, const uint16_t* Vb, int key0, int last,
                                         int h, float c, const LaneOffsets<HS>& L,
                                         const u32x4 (&qf)[HS / 16], DecState<HS>& st) {
  constexpr int KSTEP = HS / 16, DB = HS / 32;
  f32x16 s[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    s[kh] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks) s[kh] = E::mfma(op_nat<HS>(Kb, L, kh * 32, ks), qf[ks], s[kh]);
  }
  // Register i of s[kh] is key key0 + kh*32 + 16*(i/8) + 8h + i%8.
  if (MASK) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + kh * 32 + 16 * (i >> 3) + 8 * h + (i & 7) > last) s[kh][i] = -INFINITY;
  }
  float mh[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    mh[kh] = fmaxf(s[kh][0], s[kh][1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mh[kh] = fmaxf(fmaxf(mh[kh], s[kh][i]), s[kh][i + 1]);
  }
  const float mt = halves_max(fmaxf(mh[0], mh[1]));
  // Lazy rescale as in the forward (the reference max moves only when the
  // weights would exceed 2^8); a row still at m = -inf takes any finite max.
  const bool grow = mt > st.m && (st.m == -INFINITY || (mt - st.m) * c > 8.f);
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float alpha = grow ? __builtin_amdgcn_exp2f((st.m - mt) * c) : 1.f;  // -inf -> 0
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) st.oacc[db] *= alpha;
    st.m = grow ? mt : st.m;
  }
  // A row with no visible key so far has every score at -inf: weights 0.
  const float mc = st.m == -INFINITY ? 0.f : st.m * c;
  u32x4 pf[2][2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kh][8 * t + 2 * e], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kh][8 * t + 2 * e + 1], c, -mc));
        pf[kh][t][e] = E::pack(p0, p1);
        st.l += p0 + p1;
      }
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        st.oacc[db] = E::mfma(op_tr<HS>(Vb, L, kh * 32 + 16 * t, db), pf[kh][t], st.oacc[db]);
}

// Partials: opart [BH][nsplit][Tq][HS] float32 (normalised output of the
// split), lpart [BH][nsplit][Tq] float32 (natural log-sum-exp of the split's
// scores, -inf when the row saw none of its keys).
// DIRECT (one split): the workgroup's result is the final one; it writes o
// (16-bit, layout lo) and lse instead of partials.
template <class E, int HS, bool STRIDED, bool DIRECT, int NW>
__global__ __launch_bounds__(64 * NW) void dec16_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   float* __restrict__ opart,
                                                   float* __restrict__ lpart,
                                                   uint16_t* __restrict__ o,
                                                   float* __restrict__ lse, int H, int Tq,
                                                   int Tk, int nqb, int nsplit, int tps,
                                                   float scale, Layout lq, Layout lk, Layout lo) {
  constexpr int KSTEP = HS / 16, DB = HS / 32;
  // Per wavefront: a K ring and a V ring of two tiles; after the loop the same
  // memory holds the wavefronts' states for the merge.
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NW][2][kBN * HS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NW][2][kBN * HS];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int sp = int(blockIdx.x) % nsplit;
  const int qb = (int(blockIdx.x) / nsplit) % nqb;
  const int bh = int(blockIdx.x) / (nsplit * nqb);
  const int off = Tk - Tq;
  const int row = qb * 32 + n;
  const int last = off + row;  // newest key this lane's query sees
  // Key tiles any query of the block sees, and this split's share of them.
  const int kmax = off + min(qb * 32 + 31, Tq - 1);
  // This wavefront's tiles: t0 + w, t0 + w + NW, ... below t1.
  const int t0 = sp * tps + w, t1 = min(kmax / kBN + 1, sp * tps + tps);
  const int ntw = t0 < t1 ? (t1 - t0 + NW - 1) / NW : 0;

  const int rq = STRIDED ? int(lq.st) : HS, rk = STRIDED ? int(lk.st) : HS;
  const rsrc_t wq = make_rsrc(q + slice_offset(lq, bh, H), slice_span_bytes(lq, Tq, HS, 2));
  const int64_t kbase = slice_offset(lk, bh, H);
  const uint32_t kbytes = slice_span_bytes(lk, Tk, HS, 2);
  const rsrc_t wk = make_rsrc(k + kbase, kbytes), wv = make_rsrc(v + kbase, kbytes);

  DecState<HS> st;
#pragma unroll
  for (int db = 0; db < DB; ++db) st.oacc[db] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;

  if (ntw > 0) {
    const float c = scale * kLog2e;
    const LaneOffsets<HS> L(lane);
    dma_tile<HS, kBN, 1>(wk, t0 * kBN, rk, Ks[w][0], 0, lane);
    dma_tile<HS, kBN, 1>(wv, t0 * kBN, rk, Vs[w][0], 0, lane);
    // Q^T as the MFMA B operand (rows past Tq read as zero).
    u32x4 qf[KSTEP];
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks)
      qf[ks] = bload16(wq, uint32_t(row * rq + 16 * ks + 8 * h) * 2);
    // The rings are private to the wavefront: waiting for its own LDS DMA
    // is enough (no workgroup barrier inside the loop).
    wait_vmem();
    __builtin_amdgcn_wave_barrier();
    auto step = [&](int i, auto bufc) {
      constexpr int buf = decltype(bufc)::value;
      const int t = t0 + i * NW;
      if (i + 1 < ntw) {
        dma_tile<HS, kBN, 1>(wk, (t + NW) * kBN, rk, Ks[w][buf ^ 1], 0, lane);
        dma_tile<HS, kBN, 1>(wv, (t + NW) * kBN, rk, Vs[w][buf ^ 1], 0, lane);
      }
      const int key0 = t * kBN;
      if (key0 + kBN - 1 > off + qb * 32)  // some key may lie past some query
        dec_tile<E, HS, true>(Ks[w][buf], Vs[w][buf], key0, last, h, c, L, qf, st);
      else
        dec_tile<E, HS, false>(Ks[w][buf], Vs[w][buf], key0, last, h, c, L, qf, st);
      wait_vmem();
      __builtin_amdgcn_wave_barrier();
    };
    ring_loop<2>(ntw, step);
  }
  if constexpr (NW > 1) {
    // Merge the wavefronts' states: each writes its max (m, raw score units;
    // -inf if it saw none of the row's keys), sum l and unnormalised output
    // rows to LDS, then every thread combines a pair of output elements.
    constexpr int RS = HS + 4;  // padded row of the output state (floats)
    float* const mst = reinterpret_cast<float*>(&Ks[0][0][0]);       // [NW][32]
    float* const lst = mst + NW * 32;                                 // [NW][32]
    float* const ost = lst + NW * 32;                                 // [NW][32][RS]
    static_assert(sizeof(float) * NW * 32 * (RS + 2) <= sizeof(Ks), "merge state fits");
    const float lw = halves_sum(st.l);
    __syncthreads();  // every wavefront is done with its tiles
    if (h == 0) {
      mst[w * 32 + n] = st.m;
      lst[w * 32 + n] = lw;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(ost + (w * 32 + n) * RS + db * 32 + 8 * g + 4 * h) =
            f32x4{st.oacc[db][4 * g], st.oacc[db][4 * g + 1], st.oacc[db][4 * g + 2],
                  st.oacc[db][4 * g + 3]};
    __syncthreads();
    const float c = scale * kLog2e;
    for (int idx = threadIdx.x; idx < 32 * HS / 2; idx += 64 * NW) {
      const int r = idx / (HS / 2), d = 2 * (idx % (HS / 2));
      float M = -INFINITY;
#pragma unroll
      for (int u = 0; u < NW; ++u) M = fmaxf(M, mst[u * 32 + r]);
      float Ls = 0.f, a0 = 0.f, a1 = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int u = 0; u < NW; ++u) {
          const float wt = __builtin_amdgcn_exp2f((mst[u * 32 + r] - M) * c);  // -inf -> 0
          Ls += wt * lst[u * 32 + r];
          a0 = fmaf(wt, ost[(u * 32 + r) * RS + d], a0);
          a1 = fmaf(wt, ost[(u * 32 + r) * RS + d + 1], a1);
        }
      }
      const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
      const int rr = qb * 32 + r;
      if constexpr (DIRECT) {  // split 0 holds key 0, seen by every query: Ls > 0
        const rsrc_t wo = make_rsrc(o + slice_offset(lo, bh, H), slice_span_bytes(lo, Tq, HS, 2));
        const int ro = STRIDED ? int(lo.st) : HS;
        __builtin_amdgcn_raw_buffer_store_b32(E::pack(a0 * inv, a1 * inv), wo,
                                              uint32_t(rr * ro + d) * 2, 0, 0);
        if (lse != nullptr && d == 0)
          bstoref(make_rsrc(lse + long(bh) * Tq, uint32_t(Tq) * 4), uint32_t(rr) * 4,
                  M * scale + logf(Ls));
      } else {
        const long pbase = (long(bh) * nsplit + sp) * Tq;
        const rsrc_t wp = make_rsrc(opart + pbase * HS, uint32_t(Tq) * HS * 4);
        bstore8(wp, uint32_t(rr * HS + d) * 4,
                u32x2{__float_as_uint(a0 * inv), __float_as_uint(a1 * inv)});
        if (d == 0)
          bstoref(make_rsrc(lpart + pbase, uint32_t(Tq) * 4), uint32_t(rr) * 4,
                  Ls > 0.f ? M * scale + logf(Ls) : -INFINITY);
      }
    }
    return;
  }

  // O^T register i of lane (n, h): column d = db*32 + 8*(i/4) + 4h + i%4 of
  // this lane's query.  Rows past Tq are dropped by the buffer bounds.
  const float lt = halves_sum(st.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if constexpr (DIRECT) {  // split 0 holds key 0, seen by every query: lt > 0
    const rsrc_t wo = make_rsrc(o + slice_offset(lo, bh, H), slice_span_bytes(lo, Tq, HS, 2));
    const int ro = STRIDED ? int(lo.st) : HS;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t off = uint32_t(row * ro + db * 32 + 8 * g + 4 * h) * 2;
        bstore8(wo, off, u32x2{E::pack(st.oacc[db][4 * g] * inv, st.oacc[db][4 * g + 1] * inv),
                               E::pack(st.oacc[db][4 * g + 2] * inv,
                                       st.oacc[db][4 * g + 3] * inv)});
      }
    if (lse != nullptr && h == 0)
      bstoref(make_rsrc(lse + long(bh) * Tq, uint32_t(Tq) * 4), uint32_t(row) * 4,
              st.m * scale + logf(lt));
    return;
  }
  // Normalised partial output and log-sum-exp of the split.
  const long pbase = (long(bh) * nsplit + sp) * Tq;
  const rsrc_t wo = make_rsrc(opart + pbase * HS, uint32_t(Tq) * HS * 4);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t o4 = uint32_t(row * HS + db * 32 + 8 * g + 4 * h) * 4;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, f32x4{st.oacc[db][4 * g] * inv, st.oacc[db][4 * g + 1] * inv,
                                          st.oacc[db][4 * g + 2] * inv,
                                          st.oacc[db][4 * g + 3] * inv}),
          wo, o4, 0, 0);
    }
  if (h == 0)
    bstoref(make_rsrc(lpart + pbase, uint32_t(Tq) * 4), uint32_t(row) * 4,
            lt > 0.f ? st.m * scale + logf(lt) : -INFINITY);
}

// One new token (Tq = 1): the query is the newest position, so it sees every
// kept key (no mask), and an MFMA tile would leave 31 of its 32 query rows
// idle.  Vector arithmetic streams K and V instead.  Workgroup (b, h, split)
// has NW wavefronts, each taking a contiguous run of the split's keys.  A key
// row is read by LPK = HS/8 lanes (16 bytes each), so one load instruction
// covers KPI = 64/LPK consecutive keys; the lanes of a key add their partial
// dot products (xor shuffles) and each group of LPK lanes keeps its own
// online softmax state (max m in base-2 score units, sum l) and its 8 output
// columns, for the keys g, g + KPI, ... of the run.  U iterations of loads
// are in flight together.  The groups merge by xor shuffles, the wavefronts
// through LDS; the result is o and lse (DIRECT) or the split's normalised
// partial output and log-sum-exp, merged by dec16_combine.
template <class E, int HS, bool STRIDED, bool DIRECT, int NW>
__global__ __launch_bounds__(64 * NW) void dec1_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       float* __restrict__ opart,
                                                       float* __restrict__ lpart,
                                                       uint16_t* __restrict__ o,
                                                       float* __restrict__ lse, int H, int Tk,
                                                       int nsplit, int kps, float scale,
                                                       Layout lq, Layout lk, Layout lo) {
  constexpr int LPK = HS / 8, KPI = 64 / LPK, U = 4;
  __shared__ float sm[NW], sl[NW];
  __shared__ __attribute__((aligned(16))) float so[NW][HS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane / LPK, cc = lane % LPK;
  const int sp = int(blockIdx.x) % nsplit, bh = int(blockIdx.x) / nsplit;
  const int k0 = sp * kps, k1 = min(Tk, k0 + kps);
  const int per = ((k1 - k0 + NW - 1) / NW + KPI - 1) / KPI * KPI;  // keys per wavefront
  const int a = k0 + w * per, b = min(k1, a + per);
  const int rk = STRIDED ? int(lk.st) : HS;
  const int64_t kbase = slice_offset(lk, bh, H);
  const uint32_t kbytes = slice_span_bytes(lk, Tk, HS, 2);
  const rsrc_t wk = make_rsrc(k + kbase, kbytes), wv = make_rsrc(v + kbase, kbytes);
  const float c = scale * kLog2e;
  // This lane's 8 query elements, scaled into base-2 score units.
  const u32x4 qr = bload16(make_rsrc(q + slice_offset(lq, bh, H), HS * 2), uint32_t(cc * 16));
  float qf[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    qf[2 * e] = E::lo(qr[e]) * c;
    qf[2 * e + 1] = E::hi(qr[e]) * c;
  }
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // Batches of U iterations; the next batch's loads are issued before the
  // current one is computed (rows past the slice read as zero and are masked).
  auto load = [&](int base, u32x4 (&kr)[U], u32x4 (&vr)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = uint32_t((base + u * KPI + g) * rk + cc * 8) * 2;
      kr[u] = bload16(wk, off);
      vr[u] = bload16(wv, off);
    }
  };
  auto consume = [&](int base, const u32x4 (&kr)[U], const u32x4 (&vr)[U]) {
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t = fmaf(qf[2 * e], E::lo(kr[u][e]), t);
        t = fmaf(qf[2 * e + 1], E::hi(kr[u][e]), t);
      }
#pragma unroll
      for (int off = LPK / 2; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
      s[u] = base + u * KPI + g < b ? t : -INFINITY;
    }
    float mb = s[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mb = fmaxf(mb, s[u]);
    if (mb > m) {  // m = -inf at first: alpha = 0
      const float al = __builtin_amdgcn_exp2f(m - mb);
      l *= al;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= al;
      m = mb;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = s[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[u] - m);
      l += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(p, E::lo(vr[u][e]), acc[2 * e]);
        acc[2 * e + 1] = fmaf(p, E::hi(vr[u][e]), acc[2 * e + 1]);
      }
    }
  };
  constexpr int STEP = KPI * U;
  u32x4 ka[U], va[U], kb[U], vb[U];
  if (a < b) load(a, ka, va);
  for (int base = a; base < b; base += 2 * STEP) {
    if (base + STEP < b) load(base + STEP, kb, vb);
    consume(base, ka, va);
    if (base + STEP >= b) break;
    if (base + 2 * STEP < b) load(base + 2 * STEP, ka, va);
    consume(base + STEP, kb, vb);
  }
  // Merge the lane groups (a group that saw no key has m = -inf, l = 0).
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64), l2 = __shfl_xor(l, off, 64);
    const float M = fmaxf(m, m2);
    const float a1 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
    const float a2 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a1 + __shfl_xor(acc[e], off, 64) * a2;
    m = M;
  }
  if (lane == 0) {
    sm[w] = m;
    sl[w] = l;
  }
  if (g == 0) {
    *reinterpret_cast<f32x4*>(&so[w][cc * 8]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(&so[w][cc * 8 + 4]) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
  __syncthreads();
  // Merge the wavefronts: thread t < HS/2 finishes columns 2t, 2t+1.  The
  // split holds at least one key, so M is finite and L > 0.
  if (int(threadIdx.x) < HS / 2) {
    const int d = 2 * int(threadIdx.x);
    float M = sm[0];
#pragma unroll
    for (int u = 1; u < NW; ++u) M = fmaxf(M, sm[u]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const float wt = __builtin_amdgcn_exp2f(sm[u] - M);  // -inf -> 0
      L = fmaf(wt, sl[u], L);
      o0 = fmaf(wt, so[u][d], o0);
      o1 = fmaf(wt, so[u][d + 1], o1);
    }
    const float inv = 1.f / L;
    const float ls = (M + log2f(L)) * kLn2;  // natural log-sum-exp
    if constexpr (DIRECT) {
      uint16_t* orow = o + slice_offset(lo, bh, H);
      *reinterpret_cast<uint32_t*>(orow + d) = E::pack(o0 * inv, o1 * inv);
      if (lse != nullptr && d == 0) lse[bh] = ls;
    } else {
      float* op = opart + (long(bh) * nsplit + sp) * HS;
      *reinterpret_cast<float2*>(op + d) = float2{o0 * inv, o1 * inv};
      if (d == 0) lpart[long(bh) * nsplit + sp] = ls;
    }
  }
}

// One wavefront per (b, h, query): merge the splits, store o (16-bit, round
// to nearest even) and lse.  Lane j holds elements 2j, 2j+1 of the row.
template <class E, int HS>
__global__ __launch_bounds__(256) void dec16_combine(const float* __restrict__ opart,
                                                     const float* __restrict__ lpart,
                                                     uint16_t* __restrict__ o,
                                                     float* __restrict__ lse, int BH, int H,
                                                     int Tq, int nsplit, Layout lo) {
  const int lane = threadIdx.x & 63;
  const long gid = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gid >= long(BH) * Tq) return;  // uniform per wavefront
  const int bh = int(gid / Tq), row = int(gid % Tq);
  const float* lp = lpart + long(bh) * nsplit * Tq + row;
  // The splits' lse values are read across lanes (one load per lane, not one
  // dependent load per split), then reduced over the wavefront.
  float M = -INFINITY;
  for (int s = lane; s < nsplit; s += 64) M = fmaxf(M, lp[long(s) * Tq]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  // Split 0 holds key 0, which every query sees: M is finite.
  float Lsum = 0.f;
  for (int s = lane; s < nsplit; s += 64) Lsum += expf(lp[long(s) * Tq] - M);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) Lsum += __shfl_xor(Lsum, off, 64);
  // Weighted sum of the partial rows; the loop is unrolled so the loads of
  // several splits are in flight together.
  float a0 = 0.f, a1 = 0.f;
  const float* op = opart + (long(bh) * nsplit * Tq + row) * HS + 2 * lane;
  const bool act = 2 * lane < HS;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float w = expf(lp[long(s) * Tq] - M);  // exp(-inf) = 0 for an empty split
    if (act) {
      const float2 x = *reinterpret_cast<const float2*>(op + long(s) * Tq * HS);
      a0 = fmaf(w, x.x, a0);
      a1 = fmaf(w, x.y, a1);
    }
  }
  const float inv = 1.f / Lsum;
  if (2 * lane < HS) {
    uint16_t* orow = o + slice_offset(lo, bh, H) + int64_t(row) * lo.st;
    *reinterpret_cast<uint32_t*>(orow + 2 * lane) = E::pack(a0 * inv, a1 * inv);
  }
  if (lse != nullptr && lane == 0) lse[long(bh) * Tq + row] = M + logf(Lsum);
}

template <class E, int HS>
hipError_t dec16_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                        float* lse, int BH, int H, int Tq, int Tk, float scale, Layout lq,
                        Layout lk, Layout lo, float* opart, float* lpart, const DecodeSplit& ds,
                        hipStream_t s) {
  const bool strided = !(is_contiguous(lq, H, Tq, HS) && is_contiguous(lk, H, Tk, HS) &&
                         is_contiguous(lo, H, Tq, HS));
  const dim3 grid(unsigned(BH * ds.nqb * ds.nsplit));
  const bool direct = ds.nsplit == 1;
  if (ds.kps > 0) {  // one new token: the vector-ALU kernel
    constexpr int NW = GATTN_DEC1_NW;
    auto k1 = strided ? (direct ? dec1_kernel<E, HS, true, true, NW> : dec1_kernel<E, HS, true, false, NW>)
                      : (direct ? dec1_kernel<E, HS, false, true, NW>
                                : dec1_kernel<E, HS, false, false, NW>);
    hipError_t e = launch(k1, grid, dim3(64 * NW), s, q, k, v, opart, lpart, o, lse, H, Tk,
                          ds.nsplit, ds.kps, scale, lq, lk, lo);
    if (e != hipSuccess || direct) return e;
    return launch(dec16_combine<E, HS>, dim3(unsigned((BH + 3) / 4)), dim3(256), s, opart, lpart,
                  o, lse, BH, H, Tq, ds.nsplit, lo);
  }
  auto pick = [&](auto nwc) {
    constexpr int NW = decltype(nwc)::value;
    return strided ? (direct ? dec16_kernel<E, HS, true, true, NW>
                             : dec16_kernel<E, HS, true, false, NW>)
                   : (direct ? dec16_kernel<E, HS, false, true, NW>
                             : dec16_kernel<E, HS, false, false, NW>);
  };
  auto kern = ds.nw == 4 ? pick(std::integral_constant<int, 4>{})
                         : pick(std::integral_constant<int, 1>{});
  hipError_t e = launch(kern, grid, dim3(64 * ds.nw), s, q, k, v, opart, lpart, o, lse, H, Tq, Tk,
                        ds.nqb, ds.nsplit, ds.tps, scale, lq, lk, lo);
  if (e != hipSuccess || direct) return e;
  const long rows = long(BH) * Tq;
  return launch(dec16_combine<E, HS>, dim3(unsigned((rows + 3) / 4)), dim3(256), s, opart, lpart,
                o, lse, BH, H, Tq, ds.nsplit, lo);
}

}  // namespace

hipError_t h16_fwd_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                          float* lse, int BH, int H, int Tq, int Tk, int hs, float scale,
                          Layout lq, Layout lk, Layout lo, float* opart, float* lpart,
                          const DecodeSplit& ds, bool f16, hipStream_t s) {
  if (f16) {
    if (hs == 64)
      return dec16_launch<F16, 64>(q, k, v, o, lse, BH, H, Tq, Tk, scale, lq, lk, lo, opart,
                                   lpart, ds, s);
    return dec16_launch<F16, 32>(q, k, v, o, lse, BH, H, Tq, Tk, scale, lq, lk, lo, opart, lpart,
                                 ds, s);
  }
  if (hs == 64)
    return dec16_launch<Bf16, 64>(q, k, v, o, lse, BH, H, Tq, Tk, scale, lq, lk, lo, opart, lpart,
                                  ds, s);
  return dec16_launch<Bf16, 32>(q, k, v, o, lse, BH, H, Tq, Tk, scale, lq, lk, lo, opart, lpart,
                                ds, s);
}

}  // namespace gattn
