// Internal declarations shared by the gattn kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <tuple>

#include "philox.h"

namespace gattn {

// Launch a __global__ function through hipLaunchKernel so that the launch
// status comes back directly (no reliance on the thread's sticky last error).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
  void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply(
      [&](auto&... x) {
        int n = 0;
        ((argv[n++] = static_cast<void*>(&x)), ...);
      },
      vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, 0, stream);
}

// Element strides of a (B, H, T, hs) tensor whose hs elements are contiguous:
// element (b, h, t, d) sits at b*sb + h*sh + t*st + d.  The contiguous layout
// is {H*T*hs, T*hs, hs}; the fused projection output (B, T, 3C) read as q (or
// k, v at +C, +2C elements) is {T*3C, hs, 3C}; a (B, T, C) output is
// {T*C, hs, C}.
struct Layout {
  int64_t sb, sh, st;
};
inline Layout contiguous_layout(int H, int T, int hs) {
  return Layout{int64_t(H) * T * hs, int64_t(T) * hs, hs};
}
// Offset (elements) of slice (b, h) = (bh / H, bh % H).
__host__ __device__ inline int64_t slice_offset(const Layout& l, int bh, int H) {
  return int64_t(bh / H) * l.sb + int64_t(bh % H) * l.sh;
}
inline bool is_contiguous(const Layout& l, int H, int T, int hs) {
  const Layout c = contiguous_layout(H, T, hs);
  return l.sb == c.sb && l.sh == c.sh && l.st == c.st;
}
inline bool all_contiguous(int H, int T, int hs, const Layout& a, const Layout& b,
                           const Layout& c) {
  return is_contiguous(a, H, T, hs) && is_contiguous(b, H, T, hs) && is_contiguous(c, H, T, hs);
}
// Bytes spanned by one slice: rows 0 .. T-1 of hs elements of `esize` bytes.
__host__ __device__ inline uint32_t slice_span_bytes(const Layout& l, int T, int hs, int esize) {
  return uint32_t((int64_t(T - 1) * l.st + hs) * esize);
}

// Split of the key range for the forward of the newest Tq tokens (decode):
// nqb 32-query blocks; each block's key tiles (64 keys) are divided among
// nsplit workgroups of tps tiles, and a workgroup's tiles among its nw
// wavefronts (which merge through LDS).  A block with one tile, or 1024
// blocks, runs one single-wavefront workgroup per block.  Otherwise nw =
// GATTN_DEC_NW; when the blocks alone give at least GATTN_DEC_DIRECT_WAVES
// wavefronts there is no split (one launch, no workspace); else the key range
// is split so that about 2048 wavefronts stream it, every split keeping at
// least nw tiles.  The workspace size and the launch both derive from this
// one function.
#ifndef GATTN_DEC_NW
#define GATTN_DEC_NW 4
#endif
#ifndef GATTN_DEC_DIRECT_WAVES
#define GATTN_DEC_DIRECT_WAVES 512
#endif
//
// One new token (Tq = 1) takes the vector-ALU path instead: workgroups of
// GATTN_DEC1_NW wavefronts, each streaming a contiguous run of the
// workgroup's kps keys; no split when the heads give 1024 wavefronts, else
// about 2048 wavefronts with at least 64 keys each.
#ifndef GATTN_DEC1_NW
#define GATTN_DEC1_NW 8
#endif
struct DecodeSplit {
  int nqb, nsplit, tps, nw;
  int kps;  // one-token path: keys per split (0 on the MFMA path)
};
inline DecodeSplit decode_split(int BH, int Tq, int Tk) {
  DecodeSplit d;
  d.kps = 0;
  if (Tq == 1) {
    d.nqb = 1;
    d.tps = 0;
    d.nw = GATTN_DEC1_NW;
    const long waves = long(BH) * d.nw;
    long ns = 1;
    if (waves < 1024) {
      ns = (2048 + waves - 1) / waves;
      const long cap = (Tk + 64L * d.nw - 1) / (64L * d.nw);  // >= 64 keys per wavefront
      ns = ns > cap ? cap : ns;
      ns = ns < 1 ? 1 : ns;
    }
    d.kps = int((Tk + ns - 1) / ns);
    d.nsplit = (Tk + d.kps - 1) / d.kps;
    return d;
  }
  d.nqb = (Tq + 31) / 32;
  const int ntiles = (Tk + 63) / 64;
  const long blocks = long(BH) * d.nqb;
  d.tps = ntiles;
  d.nsplit = 1;
  d.nw = 1;
  if (ntiles < 2 || blocks >= 1024) return d;
  d.nw = GATTN_DEC_NW;
  if (blocks * d.nw >= GATTN_DEC_DIRECT_WAVES) return d;
  long want = (2048 + blocks * d.nw - 1) / (blocks * d.nw);
  const long cap = ntiles / d.nw > 0 ? ntiles / d.nw : 1;
  want = want > cap ? cap : want;
  d.tps = int((ntiles + want - 1) / want);
  d.nsplit = (ntiles + d.tps - 1) / d.tps;
  return d;
}
// Decode workspace: [opart BH*nsplit*Tq*hs f32][lpart BH*nsplit*Tq f32], each
// part on a 256-byte boundary.
inline size_t decode_opart_bytes(int BH, int Tq, int hs, const DecodeSplit& d) {
  return (sizeof(float) * size_t(BH) * d.nsplit * Tq * hs + 255) & ~size_t(255);
}
inline size_t decode_lpart_bytes(int BH, int Tq, const DecodeSplit& d) {
  return (sizeof(float) * size_t(BH) * d.nsplit * Tq + 255) & ~size_t(255);
}

// Backward workspace: [D = rowsum(dO * O)][L2 = lse * log2(e)], each float32
// (B, H, T) and starting on a 256-byte boundary.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t ws_part_bytes(int B, int H, int T) {
  return align256(sizeof(float) * size_t(B) * H * T);
}
// Keep-bit blocks of the 16-bit backward with dropout: per (b, h) slice,
// ng x ng blocks of 8 bytes (ng = ceil(T / 8); block (query octet, key
// group), byte e = query 8 * octet + e, bit r = key 8 * group + r).  The
// kernels address one slice's blocks with 32-bit offsets: kKeepMaxGroups
// bounds ng.
constexpr int64_t kKeepMaxGroups = 16383;
inline size_t ws_keep_bytes(int B, int H, int T) {
  const size_t ng = (size_t(T) + 7) / 8;
  return align256(size_t(B) * H * ng * ng * 8);
}

// ---- float32 path (any hs <= 128, any T; wave per row; deterministic) ----
// li: layout of q, k, v; lo: of o, dO; lg: of dq, dk, dv.  lse, D and L2 are
// contiguous (B, H, T).
// f32_fwd: Tq queries against Tk >= Tq keys, query i seeing keys
// j <= Tk - Tq + i (Tq = Tk: the causal forward); q in layout lq, k and v in lk.
// dr: dropout on the weights (dr.thr = 0: none), as in philox.h.
hipError_t f32_fwd(const float* q, const float* k, const float* v, float* o, float* lse, int BH,
                   int H, int Tq, int Tk, int hs, float scale, Layout lq, Layout lk, Layout lo,
                   const Dropout& dr, hipStream_t s);
hipError_t f32_bwd_pre(const float* o, const float* dO, const float* lse, float* D, float* L2,
                       int BH, int H, int T, int hs, Layout lo, hipStream_t s);
hipError_t f32_bwd_dkdv(const float* q, const float* k, const float* v, const float* dO,
                        const float* D, const float* L2, float* dk, float* dv, int BH, int H,
                        int T, int hs, float scale, Layout li, Layout lo, Layout lg,
                        const Dropout& dr, hipStream_t s);
hipError_t f32_bwd_dq(const float* q, const float* k, const float* v, const float* dO,
                      const float* lse, const float* D, float* dq, int BH, int H, int T, int hs,
                      float scale, Layout li, Layout lo, Layout lg, const Dropout& dr,
                      hipStream_t s);

// ---- 16-bit path: bf16 (f16 = false) or fp16 (f16 = true), hs in {32, 64}; MFMA ----
// keep: with dropout, NULL or the keep-bit blocks (ws_keep_bytes) to store
// the decisions in for the backward.
hipError_t h16_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                   float* lse, uint64_t* keep, int BH, int H, int T, int hs, float scale,
                   Layout li, Layout lo, const Dropout& dr, bool f16, hipStream_t s);
// Forward of the newest Tq tokens against Tk >= Tq keys, split over the key
// range (partials in opart / lpart, then merged into o and lse).
hipError_t h16_fwd_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                          float* lse, int BH, int H, int Tq, int Tk, int hs, float scale,
                          Layout lq, Layout lk, Layout lo, float* opart, float* lpart,
                          const DecodeSplit& ds, bool f16, hipStream_t s);
// Diagnostic loop of bf16 MFMAs: blocks workgroups of 4 wavefronts, each
// wavefront iters x 8 MFMAs of 32x32x16; one float per wavefront into sink.
hipError_t mfma_loop(float* sink, int blocks, int iters, hipStream_t s);
hipError_t issue_probe(float* sink, int blocks, int mfma_iters, int valu_iters, int kind, int roles,
                       hipStream_t s);
// Keep decisions (bytes, 1 = kept) of every (b*H + h, i, j), j and i < T.
hipError_t dropout_mask(uint8_t* keep, int BH, int T, const Dropout& dr, hipStream_t s);
hipError_t h16_bwd_pre(const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                       float* L2, int BH, int H, int T, int hs, Layout lo, bool f16,
                       hipStream_t s);
// keep: with dropout (dr.thr != 0) the keep-bit blocks, ws_keep_bytes(BH, T)
// bytes: written by h16_bwd_dq (or, keep_stored, already written by the
// forward and read by h16_bwd_dq too), read by h16_bwd_dkdv; unused otherwise.
hipError_t h16_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* dO, const float* D, const float* L2,
                        const uint64_t* keep, uint16_t* dk, uint16_t* dv, int BH, int H, int T,
                        int hs, float scale, Layout li, Layout lo, Layout lg, const Dropout& dr,
                        bool f16, hipStream_t s);
hipError_t h16_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* o, const uint16_t* dO, const float* lse, float* D,
                      float* L2, uint64_t* keep, bool keep_stored, uint16_t* dq, int BH, int H,
                      int T, int hs, float scale, Layout li, Layout lo, Layout lg,
                      const Dropout& dr, bool f16, hipStream_t s);

}  // namespace gattn
