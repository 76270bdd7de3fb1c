// 128-point Walsh-Hadamard butterflies on one block held by 16 consecutive
// lanes, 8 contiguous elements per lane (element 8 * sub + e in v[e] of lane
// `sub`).  xxqk.cn/news/652513 §2 computes the transform as log2(n) rounds of
// (a + b, a - b) butterflies: here the three rounds over element bits 0-2 run
// inside a lane and the four over element bits 3-6 pair lanes (lane ^ 1, 2, 4,
// 8) through DPP and ds_swizzle, so nothing goes through LDS.  The result is
// unnormalised (H v, not H v / sqrt(128)).  All 16 lanes of a block must run
// it together.
#pragma once

#include "tb_common.h"

namespace tb {

constexpr float kInvSqrt128 = 0.08838834764831845f;

// Lane pairs (sub, sub ^ MASK): the lower lane keeps v + p, the upper p - v.
// Both are p + (+-v): the sign flip is one XOR with a per-lane mask, the sum
// one add that can take p straight from the cross-lane read.
template <int MASK>
__device__ __forceinline__ void fwht_lane_round(float (&v)[8], int sub) {
  const uint32_t flip = (sub & MASK) != 0 ? 0x80000000u : 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = xor_lane<MASK>(v[e]);
    v[e] = p + __uint_as_float(__float_as_uint(v[e]) ^ flip);
  }
}

__device__ __forceinline__ void fwht128_lanes(float (&v)[8], int sub) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const float a = v[e], c = v[e + h];
        v[e] = a + c;
        v[e + h] = a - c;
      }
    }
  }
  fwht_lane_round<1>(v, sub);
  fwht_lane_round<2>(v, sub);
  fwht_lane_round<4>(v, sub);
  fwht_lane_round<8>(v, sub);
}

}  // namespace tb
