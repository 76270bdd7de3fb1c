// Activation operand of the dense GEMV ("act8").
//
// The dense GEMV runs on the gfx950 block-scaled matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4 with the ternary weights as fp4 (+-2, 0)
// and the activations as e4m3 with one E8M0 scale per 32 K-elements.  A bf16
// value has 8 significant bits and e4m3 has 4, so every activation is written
// as the exact sum of up to four e4m3 values on four sub-rows:
//
//   sub-row 0: level 0, high part   (sign, exponent and mantissa bits 6..4)
//   sub-row 1: level 0, low part    (mantissa bits 3..0, renormalised)
//   sub-row 2: level 1, high part
//   sub-row 3: level 1, low part
//
// Per 32-element block, level 0 holds the elements whose exponent is within
// 10 of the block's largest exponent M0, level 1 those within 10 of the largest
// exponent M1 of the rest.  Each level's scales put its largest element at
// e4m3 exponent 7, so every part is an exact normal e4m3 value and, inside the
// matrix instruction, every product lies on the 2^-13 grid below the block's
// largest product, which the hardware keeps exactly.  What is not represented:
// bf16 subnormals (|x| < 2^-126) and elements more than 20 binades below their
// block's largest; those are read as zero.
//
// Layout for B activation rows of length K (G = K / 128 groups), one buffer of
// 4 B K + B K / 8 bytes:
//   values  [B][G][4 sub-rows][4 lane groups q][32 bytes]: bytes 0-15 of lane
//           group q are K 128 g + 16 q + (0..15), bytes 16-31 are K 128 g + 64 +
//           16 q + (0..15) - the fp8 A-operand order of the instruction.
//   scales  at byte 4 B K: [B][G][4 sub-rows][4 blocks q] E8M0 codes, block q =
//           K 128 g + 32 q .. + 31.  0xFF (NaN) marks a block that held a
//           non-finite activation; its sub-row-0 element is then an e4m3 NaN.
#pragma once

#include "tb_common.h"

namespace tb {

constexpr int kActSub = 4;

__device__ __forceinline__ int quad_max(int v) {
  v = max(v, __float_as_int(xor_lane<1>(__int_as_float(v))));
  v = max(v, __float_as_int(xor_lane<2>(__int_as_float(v))));
  return v;
}

// Encode the 8 bf16 values h[e] (K = 128 g + 8 sub + e) held by lane `sub`
// (0..15) of a 128-element group and store them.  `vals` points at the group's
// 512 value bytes, `scl` at its 16 scale bytes.  All 16 lanes of the group must
// call this together (quad reductions); `store` false skips the writes.
__device__ __forceinline__ void act8_encode_store(const uint32_t (&h)[8], int sub, uint8_t* vals, uint8_t* scl,
                                                  bool store) {
  int ex[8];
  int m0 = 0, nonfinite = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ex[e] = (int)((h[e] >> 7) & 0xFFu);
    if (ex[e] == 255) nonfinite = 1;
    else m0 = max(m0, ex[e]);
  }
  m0 = quad_max(m0);
  nonfinite = quad_max(nonfinite);
  int m1 = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (ex[e] > 0 && ex[e] + 10 < m0) m1 = max(m1, ex[e]);
  m1 = quad_max(m1);

  uint32_t word[kActSub][2];
  uint32_t sc[kActSub];
#pragma unroll
  for (int lv = 0; lv < 2; ++lv) {
    const int ml = lv == 0 ? m0 : m1;
    const int s_hi = ml == 0 ? 127 : max(ml - 7, 0);
    const int s_lo = ml == 0 ? 127 : max(ml - 11, 0);
    sc[2 * lv] = (uint32_t)s_hi;
    sc[2 * lv + 1] = (uint32_t)s_lo;
    word[2 * lv][0] = word[2 * lv][1] = 0u;
    word[2 * lv + 1][0] = word[2 * lv + 1][1] = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int x = ex[e];
      const bool in = ml > 0 && x > 0 && x < 255 && x + 10 >= ml && (lv == 0 || x + 10 < m0);
      const uint32_t sgn = (h[e] >> 8) & 0x80u;
      const int ehi = x - s_hi + 7;
      uint32_t bhi = 0u, blo = 0u;
      if (in && ehi >= 1) bhi = sgn | ((uint32_t)ehi << 3) | ((h[e] >> 4) & 7u);
      const uint32_t m4 = h[e] & 0xFu;
      const int p = 31 - __builtin_clz(m4 | 1u);  // leading bit of m4 (0 when m4 <= 1)
      const int elo = x + p - s_lo;
      if (in && m4 != 0u && elo >= 1) blo = sgn | ((uint32_t)elo << 3) | ((m4 << (3 - p)) & 7u);
      word[2 * lv][e >> 2] |= bhi << (8 * (e & 3));
      word[2 * lv + 1][e >> 2] |= blo << (8 * (e & 3));
    }
  }
  if (nonfinite) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (ex[e] == 255) word[0][e >> 2] = (word[0][e >> 2] & ~(0xFFu << (8 * (e & 3)))) | (0x7Fu << (8 * (e & 3)));
    sc[0] = 0xFFu;
  }
  if (!store) return;
  // K 128 g + 8 sub .. +7 is 16-chunk c = sub / 2: lane group c % 4, half c / 4
  const int c = sub >> 1;
  const int off = (c & 3) * 32 + (c >> 2) * 16 + (sub & 1) * 8;
#pragma unroll
  for (int j = 0; j < kActSub; ++j)
    *reinterpret_cast<u32x2*>(vals + j * 128 + off) = u32x2{word[j][0], word[j][1]};
  if ((sub & 3) == 0) {
    const int q = sub >> 2;  // 32-block of this quad
#pragma unroll
    for (int j = 0; j < kActSub; ++j) scl[j * 4 + q] = (uint8_t)sc[j];
  }
}

}  // namespace tb
