// Attention dropout: the keep decisions, drawn with the Philox-4x32-10
// counter-based generator so that every kernel that needs a weight's
// decision (the forward and both backward kernels) recomputes it from the
// weight's position instead of storing a mask.
//
// Dropout probability 0.1 is the RobGPT setting ("GPT da zero", parameter
// table); it acts on the attention weights after the row softmax, and kept
// weights are multiplied by 1/(1 - p).
//
// Generator (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC 2011): ten rounds over a 4-word counter, each taking the two
// 64-bit products of words 0 and 2 with the multipliers below, xoring their
// high halves into words 1 and 3 with the round key, and moving the low
// halves; the 2-word key advances by the Weyl constants between rounds.
//
// Decision for weight (query i, key j) of slice bh = b*H + h: the block for
// counter (i, j >> 3, bh, offset) under key (seed low, seed high) yields
// eight 16-bit values, key 8g + r taking half (r & 1) (low half first) of
// word r >> 1; the weight is kept when its value is >= thr, where
// thr = round(p * 65536).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gattn {

// Dropout parameters as the kernels see them.  thr = 0 means no dropout.
struct Dropout {
  uint32_t k0, k1;  // Philox key: the seed's low and high words
  uint32_t off;     // fourth counter word (a caller-chosen stream index)
  uint32_t thr;     // a weight is kept when its 16-bit value is >= thr
  float zs;         // 65536 / (65536 - thr): the factor on kept weights
  float izs;        // 1 / zs = (65536 - thr) / 65536 (exact)
  float lzs;        // log2(zs): the backward folds zs into its exponent
};

struct Philox4 {
  uint32_t x[4];
};

// a ^ b ^ c in one instruction (v_bitop3_b32 with the truth table of a
// three-way exclusive or).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
  // The key is uniform: keep it in two scalar registers and advance it with
  // scalar adds in every call, rather than letting the compiler hoist all ten
  // round keys into 20 scalar registers for the whole kernel.
  asm volatile("" : "+s"(k0), "+s"(k1));
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t a = uint64_t(kM0) * c0;
    const uint64_t b = uint64_t(kM1) * c2;
    const uint32_t n0 = xor3(uint32_t(b >> 32), c1, k0);
    const uint32_t n2 = xor3(uint32_t(a >> 32), c3, k1);
    c1 = uint32_t(b);
    c3 = uint32_t(a);
    c0 = n0;
    c2 = n2;
    k0 += kW0;
    k1 += kW1;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// The generator block of the run of 8 keys 8g .. 8g+7 for query i.
__device__ __forceinline__ Philox4 keep_block(uint32_t i, uint32_t g, uint32_t bh,
                                              const Dropout& d) {
  return philox4x32_10(i, g, bh, d.off, d.k0, d.k1);
}

// Keep tests of the two values in one word, against thr16 = thr << 16: the
// low half (even key) and the high half (odd key), one compare each.
__device__ __forceinline__ bool keep_lo(uint32_t w, uint32_t thr16) { return (w << 16) >= thr16; }
__device__ __forceinline__ bool keep_hi(uint32_t w, uint32_t thr16) { return w >= thr16; }

// Keep test of key 8g + r of a block.
__device__ __forceinline__ bool keep_of(const Philox4& y, int r, uint32_t thr16) {
  // selects, not an indexed load: r may be a runtime value
  const uint32_t w = (r & 4) ? ((r & 2) ? y.x[3] : y.x[2]) : ((r & 2) ? y.x[1] : y.x[0]);
  return (r & 1) ? keep_hi(w, thr16) : keep_lo(w, thr16);
}

// Keep bits of the run of 8 keys 8g .. 8g+7 for query i (bit r = key 8g + r).
// Without compares: u + (65536 - thr) has bit 16 set exactly when u >= thr.
__device__ __forceinline__ uint32_t keep_bits8(uint32_t i, uint32_t g, uint32_t bh,
                                               const Dropout& d) {
  const Philox4 y = keep_block(i, g, bh, d);
  const uint32_t c = 0x10000u - d.thr;
  uint32_t bits = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (y.x[w] & 0xFFFFu) + c, hi = (y.x[w] >> 16) + c;
    bits |= ((lo >> (16 - 2 * w)) & (1u << (2 * w))) | ((hi >> (15 - 2 * w)) & (2u << (2 * w)));
  }
  return bits;
}

// Keep decision of one weight (query i, key j).
__device__ __forceinline__ bool keep_one(uint32_t i, uint32_t j, uint32_t bh, const Dropout& d) {
  return keep_of(keep_block(i, j >> 3, bh, d), int(j & 7), d.thr << 16);
}

// All ones if bit `bit` of `bits` is set, else 0 (one signed bit-field extract).
__device__ __forceinline__ uint32_t keep_mask(uint32_t bits, int bit) {
  return uint32_t(__builtin_amdgcn_sbfe(int(bits), bit, 1));
}

// x if bit `bit` of `bits` is set, else +0 (a bit mask, no compare/select).
__device__ __forceinline__ float keep_or_zero(float x, uint32_t bits, int bit) {
  return __uint_as_float(__float_as_uint(x) & keep_mask(bits, bit));
}

}  // namespace gattn
