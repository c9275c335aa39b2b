// Device helpers for the 16-bit (bf16, fp16) MFMA kernels: vector types,
// element traits (MFMA, pack, unpack), LDS tiles, LDS DMA, rings.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace gattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (x in the low half), round to nearest even
// (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ inline uint32_t pack_bf16(float x, float y) {
  bf16x2 r = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(uint32_t, r);
}

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).
// Operand layout (lane l, slot s = 0..7): A[m = l%32][k = 8*(l/32) + s],
// B[k = 8*(l/32) + s][n = l%32].  Result register i of lane l holds
// D[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ inline f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Row permutation for the A operand of a 32x32 MFMA: swapping bits 2 and 3
// of the row index makes result register i of lane l hold row
// 16*(i/8) + 8*(l/32) + i%8, so each lane's registers 8t..8t+7 cover 8
// consecutive rows: the k-slot layout of a following MFMA's operand.
__device__ inline int perm_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Element traits of the 16-bit kernels.  Both types use the same 32x32x16
// MFMA shape and operand layout (above) and the same LDS tiles; they differ in
// the MFMA opcode and in the conversions:
//   mfma(a, b, c) : D += A B with A, B packed 16-bit operands;
//   pack(x, y)    : two floats -> packed pair (x in the low half), round to
//                   nearest even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32);
//   lo(w), hi(w)  : the low / high element of a packed pair as a float.
struct Bf16 {
  __device__ static f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
    return mfma32(a, b, c);
  }
  __device__ static uint32_t pack(float x, float y) { return pack_bf16(x, y); }
  __device__ static float lo(uint32_t w) { return bf16lo(w); }
  __device__ static float hi(uint32_t w) { return bf16hi(w); }
};
struct F16 {
  __device__ static f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack(float x, float y) {
    f16x2 r = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static float lo(uint32_t w) { return float(__builtin_bit_cast(f16x2, w)[0]); }
  __device__ static float hi(uint32_t w) { return float(__builtin_bit_cast(f16x2, w)[1]); }
};

// Element type of the backward's dS products (dQ = scale dS K, dK = scale
// dS^T Q, and the row-term correction P K): fp16 for both 16-bit types.
// dS rounded to bf16 (8 significant bits) moves dQ and dK by up to
// 2^-9 |dS| |K| per term, which for inputs of twice unit variance already
// exceeds 2e-2 + 2^-8 |ref|; fp16 keeps 11 bits.  The other operand (K or Q)
// is then needed in fp16 too: for bf16 inputs it is converted, exactly for
// magnitudes in [2^-14, 65504] (smaller ones keep 2^-24 absolute precision
// as fp16 subnormals, larger ones become inf), and dS must stay below 65504.
template <class E>
struct DsOf {
  using T = F16;
  static constexpr bool kConvert = !std::is_same<E, F16>::value;
};

// Packed bf16 pair -> packed fp16 pair (round to nearest even).
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t w) { return F16::pack(bf16lo(w), bf16hi(w)); }
__device__ inline u32x4 bf16x8_to_f16x8(const u32x4& x) {
  return u32x4{bf16x2_to_f16x2(x[0]), bf16x2_to_f16x2(x[1]), bf16x2_to_f16x2(x[2]),
               bf16x2_to_f16x2(x[3])};
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ds_read_b64_tr_b16 (gfx950 LDS transpose read).  Within each group of 16
// lanes, every lane names an 8-byte segment (4 bf16); output element e of
// lane i of the group is element i%4 of the segment named by lane 4e + i/4.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ inline u32x2 ds_read_tr(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Buffer resources: raw (stride 0) buffers whose size bounds every access in
// hardware.  Loads past `bytes` return zero and stores past it are dropped,
// so row tails need no branches.  The fourth descriptor word is the gfx9
// raw-buffer format (32-bit data format, no swizzle).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
__device__ inline u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline float bloadf(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void bstore8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
__device__ inline void bstoref(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}
__device__ inline void bstore1(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(static_cast<unsigned char>(v), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles.  A tile holds rows of HS bf16 back to back (HS*2 bytes,
// no padding); the 16-byte chunk c of row r sits at chunk position
// c ^ swz(r).  The swizzle makes both access patterns below free of bank
// conflicts (64 banks x 4 bytes):
//   * MFMA operand rows (16-byte reads, 32 consecutive or perm_row-ordered
//     rows, one chunk each);
//   * transpose reads (8 bytes per lane, 4 rows x 64 bytes per 32 lanes).
// HS = 64: rows r, r+1 share swz = rot3((r >> 1) & 7), rot3 moving bit 0 to
// bit 2, so rows r and r+2 use opposite halves of the row; HS = 32:
// swz = (r >> 2) & 3.
template <int HS>
__device__ inline int swz(int r) {
  if constexpr (HS == 64) {
    const int j = (r >> 1) & 7;
    return ((j & 1) << 2) | (j >> 1);
  } else {
    return (r >> 2) & 3;
  }
}
// Element offset of (row r, column col) in a swizzled tile.
template <int HS>
__device__ inline int toff(int r, int col) {
  return r * HS + ((((col >> 3) ^ swz<HS>(r)) & (HS / 8 - 1)) << 3) + (col & 7);
}
// 16-byte MFMA operand: row r, columns col .. col+7 (col a multiple of 8).
template <int HS>
__device__ inline u32x4 tile_row16(const uint16_t* tile, int r, int col) {
  return *reinterpret_cast<const u32x4*>(tile + toff<HS>(r, col));
}

// 32x32x16 MFMA operand (lane l holds n = l%32 and k = 8*(l/32) .. +7, i.e.
// the B layout, which is also the A layout with m in place of n) read from a
// swizzled tile M[k][n] (row = k), for k0 .. k0+15 and n0 .. n0+31, with two
// transpose reads (rows +0..3 and +4..7 of each 8-row half).
template <int HS>
__device__ inline u32x4 tile_operand_tr(const uint16_t* M, int k0, int n0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int r = k0 + 8 * (g >> 1) + (j >> 2);
  const int col = n0 + 16 * (g & 1) + 4 * (j & 3);
  const u32x2 a = ds_read_tr(M + toff<HS>(r, col)), b = ds_read_tr(M + toff<HS>(r + 4, col));
  return u32x4{a[0], a[1], b[0], b[1]};
}

// Per-lane element offsets into a swizzled tile, computed once per kernel.
// The swizzle repeats every 16 rows, so a block starting at a multiple of 16
// rows only adds a compile-time constant: every LDS read in the main loops is
// (lane offset register) + (immediate).
//   nat[ks]    : row perm_row(l%32), columns 16 ks + 8 (l/32) .. +7, i.e. the
//                16-byte A (or B) operand row of a 32x32x16 MFMA whose 32
//                rows start at a multiple of 32;
//   tra/trb[db]: the two transpose reads of tile_operand_tr for k0 = 0 and
//                n0 = 32 db (add k0 * HS for a block starting at row k0).
template <int HS>
struct LaneOffsets {
  int nat[HS / 16];
  int tra[HS / 32], trb[HS / 32];
  __device__ explicit LaneOffsets(int lane) {
    const int n = lane & 31, h = lane >> 5;
    const int prow = perm_row(n);
#pragma unroll
    for (int ks = 0; ks < HS / 16; ++ks) nat[ks] = toff<HS>(prow, 16 * ks + 8 * h);
    const int g = lane >> 4, j = lane & 15;
    const int r = 8 * (g >> 1) + (j >> 2), col = 16 * (g & 1) + 4 * (j & 3);
#pragma unroll
    for (int db = 0; db < HS / 32; ++db) {
      tra[db] = toff<HS>(r, 32 * db + col);
      trb[db] = toff<HS>(r + 4, 32 * db + col);
    }
  }
};
// Natural operand of the 32-row block starting at row r0 (r0 % 32 == 0).
template <int HS>
__device__ inline u32x4 op_nat(const uint16_t* tile, const LaneOffsets<HS>& L, int r0, int ks) {
  return *reinterpret_cast<const u32x4*>(tile + r0 * HS + L.nat[ks]);
}
// Transposed operand of rows k0 .. k0+15 (k0 % 16 == 0), columns 32 db .. +31.
template <int HS>
__device__ inline u32x4 op_tr(const uint16_t* tile, const LaneOffsets<HS>& L, int k0, int db) {
  const u32x2 a = ds_read_tr(tile + k0 * HS + L.tra[db]);
  const u32x2 b = ds_read_tr(tile + k0 * HS + L.trb[db]);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// Tile load by LDS DMA (buffer_load_dwordx4 ... lds): every lane moves 16
// bytes from global memory straight into LDS at (wave's LDS base) + 16 * lane,
// with no register staging.  Lane L of DMA instruction i fills chunk position
// L % (HS/8) of tile row i*(512/HS) + L/(HS/8), so it fetches the global chunk
// that the swizzle puts there.  Rows past the buffer resource's end arrive as
// zeros.  ROWS rows starting at global row row0 of the resource, whose rows
// are `st` elements apart; the NW wavefronts of the workgroup share the
// instructions.  The caller waits (s_waitcnt vmcnt) and synchronises before
// reading the tile.
template <int HS, int ROWS, int NW>
__device__ inline void dma_tile(rsrc_t r, int row0, int st, uint16_t* tile, int w, int lane) {
  constexpr int RPI = 512 / HS;  // rows per DMA instruction (1 KB)
  constexpr int NI = ROWS / RPI;
  static_assert(NI * RPI == ROWS, "tile rows");
#pragma unroll
  for (int i = w; i < NI; i += NW) {
    const int rl = i * RPI + lane / (HS / 8);
    const int c = (lane % (HS / 8)) ^ swz<HS>(rl);
    const uint32_t off = uint32_t((row0 + rl) * st + c * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(tile + i * 512), 16, off, 0, 0, 0);
  }
}
// Converts, in place, the bf16 chunks of a tile that this wavefront's own
// dma_tile<HS, ROWS, NW> instructions wrote (lane L of instruction i: the 16
// bytes at element i*512 + 8L) to fp16.  Call after the wavefront's own wait
// for that DMA and before the barrier that publishes the tile: the chunks
// converted are exactly the ones this wavefront's wait covers, so the whole
// tile is fp16 once every wavefront has passed the barrier.
template <int HS, int ROWS, int NW>
__device__ inline void dma_tile_to_f16(uint16_t* tile, int w, int lane) {
  constexpr int NI = ROWS * HS / 512;
#pragma unroll
  for (int i = w; i < NI; i += NW) {
    u32x4* p = reinterpret_cast<u32x4*>(tile + i * 512 + 8 * lane);
    *p = bf16x8_to_f16x8(*p);
  }
}
// DMA of n32 4-byte values (n32 <= 64) from byte offset off0 of a resource
// into LDS (one instruction; lanes >= n32 idle).
__device__ inline void dma_f32(rsrc_t r, uint32_t off0, float* dst, int n32, int lane) {
  if (lane < n32)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst), 4,
                                             off0 + 4u * lane, 0, 0, 0);
}
// Wait until at most N of this wavefront's vector-memory operations (LDS DMA
// included) are outstanding; they complete in issue order.  LDS and export
// counters are left alone (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ inline void wait_vmem() { wait_vmem_n<0>(); }

// Runs step(t, std::integral_constant<int, t % NS>) for t = t0 .. min(t0+NS, n)-1,
// so that inside a step the ring buffer index is a compile-time constant
// (its LDS offsets become instruction immediates).
template <int B, int NS, class F>
__device__ inline void ring_block(int t0, int n, F& step) {
  if constexpr (B < NS) {
    if (t0 + B < n) {
      step(t0 + B, std::integral_constant<int, B>{});
      ring_block<B + 1, NS>(t0, n, step);
    }
  }
}
template <int NS, class F>
__device__ inline void ring_loop(int n, F& step) {
  for (int t0 = 0; t0 < n; t0 += NS) ring_block<0, NS>(t0, n, step);
}

// Grid order of the training kernels: tile rank r (heaviest tiles first)
// times the row length returned here, plus the head.  The dispatcher deals
// workgroups to the 8 XCDs in turn, so with a multiple of 8 every tile of head
// bh runs on XCD bh % 8 and reads that head's rows through one L2.  Whole
// heads per XCD are then ceil(BH/8) on some XCDs and floor(BH/8) on others, so
// the count is padded (padding workgroups, head >= BH, exit at once) only when
// that costs at most 8/BH <= 1/32 of balance; a smaller count that is not a
// multiple of 8 keeps the plain order, which spreads every head's tiles over
// the XCDs but balances them exactly (12 heads padded to 16: XCDs 0-3 would
// hold two heads, XCDs 4-7 one).
__host__ __device__ inline int heads_padded(int BH) {
  return BH % 8 == 0 || BH < 256 ? BH : (BH + 7) & ~7;
}

// Element offset and byte span of slice bh of a tensor: through its Layout,
// or, when STRIDED is false (contiguous (B, H, T, HS)), as bh*T*HS and T*HS*2
// without the layout's division by H.
template <int HS, bool STRIDED, class L>
__device__ inline int64_t slice_base(const L& l, int bh, int H, int T) {
  if constexpr (STRIDED) return slice_offset(l, bh, H);
  return int64_t(bh) * T * HS;
}
template <int HS, bool STRIDED, class L>
__device__ inline uint32_t slice_bytes_of(const L& l, int T) {
  if constexpr (STRIDED) return slice_span_bytes(l, T, HS, 2);
  return uint32_t(T) * HS * 2;
}

// Ring of NS LDS stages fed by DMA: before computing step t, step t+NS-1 is
// issued; after it, the caller needs step t+1 complete, i.e. at most the DMA
// of the steps after t+1 that were issued may remain outstanding.  PER is the
// number of DMA instructions one wavefront issues per step (the same for
// every wavefront).  `later` = steps issued after step t+1 (0 .. NS-2).
template <int NS, int PER>
__device__ inline void wait_ring(int later) {
  if constexpr (NS >= 4) {
    if (later >= 2) {
      wait_vmem_n<2 * PER>();
      return;
    }
  }
  if constexpr (NS >= 3) {
    if (later >= 1) {
      wait_vmem_n<PER>();
      return;
    }
  }
  wait_vmem_n<0>();
}

// Reductions across the two 32-lane halves of a wavefront (lanes l and l^32)
// with v_permlane32_swap: swap(x, x) yields the pair (x[l], x[l^32]) in every lane.
__device__ inline float halves_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float halves_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

}  // namespace gattn
