// fa_dropout.h -- the keep mask of attention dropout, regenerated wherever it
// is needed (forward, dK/dV, dQ) from a counter-based generator instead of
// being stored.
//
// Page "blog.xiaohack.org/tag/flops", section 7 (算子融合优化), lists dropout
// inside the fused softmax step.  Here it is inverted dropout of the
// normalised probabilities: a kept probability is multiplied by
// 256 / (256 - t), a dropped one is 0, and a score is dropped with
// probability t / 256.
//
// Generator: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011).  Each round multiplies counter
// words 0 and 2 by the constants M0, M1 into 64-bit products; the new words
// are (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0), and the key advances by the
// Weyl constants W0, W1 between rounds.
//
// Mapping: one call covers the 4x4 block of queries 4I..4I+3 and keys
// 4J..4J+3 of head bh, with counter (J, I, bh, offset) and key (seed low
// word, seed high word); output word a holds queries 4I+a, its byte b
// (bits 8b..8b+7) key 4J+b, and the score is kept iff that byte >= t.
//
// Register layouts: the forward and dQ kernels hold one query per lane and
// keys in runs of four registers; the dK/dV kernel holds one key per lane and
// queries in runs of four.  In both, the four lanes of a DPP quad share the
// same four blocks of a 32-wide accumulator tile, so each lane generates one
// block and the quad exchanges words (`quad_transpose`); the dK/dV layout
// first turns its block's bytes around (`byte_transpose`).
#pragma once
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// 32 x 32 -> 64-bit product with one v_mad_u64_u32.  Written as a plain
// 64-bit multiply, the compiler splits about half of the products into a
// v_mul_hi_u32 / v_mul_lo_u32 pair, two quarter-rate instructions instead of
// one (the forward with dropout measured 689 -> 659 us at the causal
// 1 x 32 x 8192 x 128 shape).  The carry-out the instruction also writes is
// discarded.
FA_DEV uint64_t mul_wide(uint32_t a, uint32_t m) {
  uint64_t p, carry;
  asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(p), "=s"(carry) : "v"(a), "s"(m));
  return p;
}

// Philox4x32 state: four counter words.
struct Philox4 {
  uint32_t x0, x1, x2, x3;
  // rounds r0 .. r1-1 (of 0 .. 9) under key (k0, k1); round r uses the key
  // advanced r times
  FA_DEV void rounds(int r0, int r1, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = r0; r < r1; ++r) {
      const uint32_t rk0 = k0 + (uint32_t)r * 0x9E3779B9u;
      const uint32_t rk1 = k1 + (uint32_t)r * 0xBB67AE85u;
      const uint64_t p0 = mul_wide(x0, 0xD2511F53u);
      const uint64_t p1 = mul_wide(x2, 0xCD9E8D57u);
      // three-input xors as one v_bitop3_b32 each (truth table 0x96)
      const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), x1, rk0, 0x96);
      const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), x3, rk1, 0x96);
      x1 = (uint32_t)p1;
      x3 = (uint32_t)p0;
      x0 = n0;
      x2 = n2;
    }
  }
  FA_DEV u32x4 words() const { return u32x4{x0, x1, x2, x3}; }
};

// Value of the same register in quad lane c^1, c^2 (DPP quad permutations
// [1,0,3,2] and [2,3,0,1]).
FA_DEV uint32_t quad_xor1(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true); }
FA_DEV uint32_t quad_xor2(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true); }

// 4x4 transpose of words over each quad of lanes: quad lane c (c = lane % 4)
// passes x[0..3] and receives y with y[i] = x[c] of quad lane i.  Two swap
// stages: words whose index differs from c in bit 0, then in bit 1, trade
// places with the lane that differs in that bit.
FA_DEV u32x4 quad_transpose(u32x4 x, int c) {
  const bool b0 = (c & 1) != 0, b1 = (c & 2) != 0;
  const uint32_t a0 = quad_xor1(x[1]), a1 = quad_xor1(x[0]), a2 = quad_xor1(x[3]), a3 = quad_xor1(x[2]);
  u32x4 y;
  y[0] = b0 ? a0 : x[0];
  y[1] = b0 ? x[1] : a1;
  y[2] = b0 ? a2 : x[2];
  y[3] = b0 ? x[3] : a3;
  const uint32_t e0 = quad_xor2(y[2]), e1 = quad_xor2(y[3]), e2 = quad_xor2(y[0]), e3 = quad_xor2(y[1]);
  u32x4 z;
  z[0] = b1 ? e0 : y[0];
  z[1] = b1 ? e1 : y[1];
  z[2] = b1 ? y[2] : e2;
  z[3] = b1 ? y[3] : e3;
  return z;
}

// In-lane 4x4 byte transpose: byte a of y[c] = byte c of x[a].  Eight
// v_perm_b32 byte selects: __builtin_amdgcn_perm(hi, lo, sel) picks result
// byte i from byte sel_i of the 8-byte value hi:lo (0..3 from lo, 4..7 from
// hi).  First the byte pairs of x0, x1 and of x2, x3 are interleaved, then the
// interleaved halves are joined.
FA_DEV u32x4 byte_transpose(u32x4 x) {
  const uint32_t lo01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);   // x0.b0 x1.b0 x0.b1 x1.b1
  const uint32_t hi01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);   // x0.b2 x1.b2 x0.b3 x1.b3
  const uint32_t lo23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  u32x4 y;
  y[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);   // x0.b0 x1.b0 x2.b0 x3.b0
  y[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  y[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  y[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
  return y;
}

// Whether the score of mask byte jj (0..3) of word w is kept.
FA_DEV bool kept(uint32_t w, int jj, uint32_t t) { return ((w >> (8 * jj)) & 0xFFu) >= t; }

}  // namespace fa
