// Register decoder of packed OPQ words, shared by the dequantize and linear
// kernels (model card "OPQ INT4 Z-Image", "技术细节 / 推理解码": a code q of a
// row with scale m stands for bf16(G_q m) with the weight's sign).
//
// A row's sixteen bf16 table entries are held as byte planes in eight
// registers; v_perm_b32 looks up four codes at a time (bytes 0..7 of a plane
// pair, the code's bit 3 choosing the pair), so one packed word (eight codes)
// becomes eight bfloat16 values with ~40 VALU instructions and no memory.
#pragma once

#include "device_common.hpp"

namespace opq {

// Byte planes of a row's sixteen bf16 table entries: lo[i] holds the low bytes
// of entries 4i..4i+3, hi[i] the high bytes.
struct RowLut {
  uint32_t lo[4];
  uint32_t hi[4];
};

__device__ __forceinline__ RowLut make_row_lut(const Levels& lv, float m) {
  RowLut t;
#pragma unroll
  for (int i = 0; i < 4; ++i) t.lo[i] = t.hi[i] = 0u;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const uint32_t e = lut_entry(lv, q, m);
    t.lo[q >> 2] |= (e & 0xFFu) << (8 * (q & 3));
    t.hi[q >> 2] |= (e >> 8) << (8 * (q & 3));
  }
  return t;
}

// The same planes from a table spread over lanes 0..15 (lane q holds L[q] in
// its low 16 bits); the result is uniform across the wave.
__device__ __forceinline__ RowLut row_lut_from_lanes(uint32_t e) {
  RowLut t;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)e, 4 * j + i);
      lo |= (v & 0xFFu) << (8 * i);
      hi |= ((v >> 8) & 0xFFu) << (8 * i);
    }
    t.lo[j] = lo;
    t.hi[j] = hi;
  }
  return t;
}

// One plane looked up for four codes (one per byte of `sel7`, bit 3 stripped);
// `mask` has 0xFF in the bytes whose code is >= 8.
__device__ __forceinline__ uint32_t plane4(const uint32_t (&p)[4], uint32_t sel7, uint32_t mask) {
  const uint32_t a = __builtin_amdgcn_perm(p[1], p[0], sel7);
  const uint32_t b = __builtin_amdgcn_perm(p[3], p[2], sel7);
  return (b & mask) | (a & ~mask);
}

// Eight bfloat16 values of one packed word in k order: out = {(k0,k1),
// (k2,k3), (k4,k5), (k6,k7)}.  `sb` holds the sign byte in bits 0..7.  With
// kPlusZero a sign bit only marks a nonzero code, so code 0 always gives +0.0
// (without it, a negative zero may come out, which no product can tell apart).
template <bool kPlusZero = true>
__device__ __forceinline__ void decode_word_ordered(uint32_t w, uint32_t sb, const RowLut& t,
                                                    uint32_t (&out)[4]) {
  const uint32_t se7 = w & 0x07070707u;
  const uint32_t so7 = (w >> 4) & 0x07070707u;
  const uint32_t w4 = w << 4;
  const uint32_t me = __builtin_amdgcn_perm(w4 << 8, w4, 0x090B080Au);
  const uint32_t mo = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
  const uint32_t lo_e = plane4(t.lo, se7, me), hi_e = plane4(t.hi, se7, me);
  const uint32_t lo_o = plane4(t.lo, so7, mo), hi_o = plane4(t.hi, so7, mo);
  // bit 7 of each byte: the code is not 0
  const uint32_t nz_e = kPlusZero ? (w & 0x0F0F0F0Fu) + 0x7F7F7F7Fu : 0xFFFFFFFFu;
  const uint32_t nz_o = kPlusZero ? ((w >> 4) & 0x0F0F0F0Fu) + 0x7F7F7F7Fu : 0xFFFFFFFFu;
  const uint32_t sge = __umul24((sb << 7) & 0x2A80u, 0x41041u);
  const uint32_t sgo = __umul24((sb << 6) & 0x2A80u, 0x41041u);
  const uint32_t hs_e = hi_e | (sge & nz_e & 0x80808080u);
  const uint32_t hs_o = hi_o | (sgo & nz_o & 0x80808080u);
  const uint32_t e02 = __builtin_amdgcn_perm(hs_e, lo_e, 0x05010400u);  // (k0, k2)
  const uint32_t e46 = __builtin_amdgcn_perm(hs_e, lo_e, 0x07030602u);  // (k4, k6)
  const uint32_t o13 = __builtin_amdgcn_perm(hs_o, lo_o, 0x05010400u);  // (k1, k3)
  const uint32_t o57 = __builtin_amdgcn_perm(hs_o, lo_o, 0x07030602u);  // (k5, k7)
  out[0] = __builtin_amdgcn_perm(o13, e02, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(o13, e02, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(o57, e46, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(o57, e46, 0x07060302u);
}

// The same eight values (k order) with fewer instructions, for the linear
// layers, where a sign on code 0 makes no difference (it may give -0.0).  The
// codes go into two selector words as (c0, c1, c4, c5) and (c2, c3, c6, c7):
// then the bit-3 masks come straight from shifted copies of the word, and
// the bf16 pairs come out in k order with one permute each.  The sign bits
// of each group move to the top of its bytes with one 24-bit multiply:
// bits (0, 1, 4, 5) of sb placed at 5, 6, 9, 10 and multiplied by
// 2^2 + 2^9 + 2^14 + 2^21 land on 7, 15, 23, 31 (the other partial products
// fall elsewhere, and their one carry stops below bit 22).  ~34 VALU.
__device__ __forceinline__ void decode_word_split(uint32_t w, uint32_t sb, const RowLut& t,
                                                  uint32_t (&out)[4]) {
  const uint32_t ev7 = w & 0x07070707u;         // low 3 bits of codes 0, 2, 4, 6
  const uint32_t od7 = (w >> 4) & 0x07070707u;  // of codes 1, 3, 5, 7
  const uint32_t a7 = __builtin_amdgcn_perm(od7, ev7, 0x06020400u);  // c0 c1 c4 c5
  const uint32_t b7 = __builtin_amdgcn_perm(od7, ev7, 0x07030501u);  // c2 c3 c6 c7
  // 0xFF in the bytes whose code is >= 8: its bit 3 (bit 4i + 3 of w) moved
  // to bit 15 or 31 of one of the two sources, which selectors 8..11 repeat
  const uint32_t ma = __builtin_amdgcn_perm(w << 8, w << 12, 0x0B090A08u);
  const uint32_t mb = __builtin_amdgcn_perm(w, w << 4, 0x0B090A08u);
  const uint32_t lo_a = plane4(t.lo, a7, ma), lo_b = plane4(t.lo, b7, mb);
  uint32_t hi_a = plane4(t.hi, a7, ma), hi_b = plane4(t.hi, b7, mb);
  // opaque: keeps each high plane one v_bfi_b32 and the sign one v_and_or_b32
  // (left free, the combiner merges the three terms into four instructions)
  asm volatile("" : "+v"(hi_a), "+v"(hi_b));
  const uint32_t sa = __umul24((sb << 5) & 0x660u, 0x204204u);
  const uint32_t sg = __umul24((sb << 3) & 0x660u, 0x204204u);
  const uint32_t hs_a = hi_a | (sa & 0x80808080u);
  const uint32_t hs_b = hi_b | (sg & 0x80808080u);
  out[0] = __builtin_amdgcn_perm(hs_a, lo_a, 0x05010400u);  // (k0, k1)
  out[1] = __builtin_amdgcn_perm(hs_b, lo_b, 0x05010400u);  // (k2, k3)
  out[2] = __builtin_amdgcn_perm(hs_a, lo_a, 0x07030602u);  // (k4, k5)
  out[3] = __builtin_amdgcn_perm(hs_b, lo_b, 0x07030602u);  // (k6, k7)
}

}  // namespace opq
