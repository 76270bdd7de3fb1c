// Decode GEMV with dense ternary weights:
//   y[b][n] = sum_g f16(scale[n][g]) * sum_{k in g} t[n][k] * x[b][k]
// (mhpq.cn/news/1159370 §4.2: read the weight bits, expand, scale, multiply).
//
// HBM bound: every weight is streamed once at 2 bits plus 1/8 bit of scale.
// The inner product runs on the matrix cores, which keeps the vector ALU for
// decoding (about one VALU op per weight, the same for batch 1 and 16):
//   * a code word holds the 8 even-k fields in its low half and the 8 odd-k
//     fields in its high half, so (word << (14 - 2f)) & 0xC000C000 is the bf16
//     pair (2 t[k], 2 t[k+1]) for field f: sign bit 15, and bit 14 alone is the
//     exponent of 2.0.  That pair lines up with the bf16 pair (x[k], x[k+1])
//     as it sits in memory, so activations feed the MFMA unchanged.
//   * v_mfma_f32_16x16x32_bf16 with A = activations (16 batch rows, unused rows
//     zero) and B = decoded weights (16 output rows): lane (i, q) supplies 8
//     consecutive K of row i, D[4q + r][i] comes back in lane (i, q).  One
//     lane's B operand for group g is two code words (K 128g + 32q .. +31), so
//     each lane loads 8 contiguous bytes of codes per group and row tile.
//   * per group the four MFMA results are scaled by f16(scale) / 2 in fp32.
// Work split: a workgroup owns TILES x 16 output rows; its KS waves split the K
// groups and reduce through LDS.  Loads run PREFETCH groups ahead.
#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

constexpr int kPrefetch = 4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int TILES>
__global__ void __launch_bounds__(512) gemv_ternary_kernel(const uint16_t* __restrict__ x, int B,
                                                            const uint32_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales, int64_t N,
                                                            int64_t K, float* __restrict__ y, int KS) {
  extern __shared__ float red[];  // [KS][TILES][4][64]
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int li = lane & 15;  // batch row of the A operand / output row of the B operand
  const int q = lane >> 4;   // which 32-wide quarter of a group this lane covers
  const int64_t G = K / kBlock;
  const int64_t row0 = (int64_t)blockIdx.x * (16 * TILES) + li;
  const int64_t gb = G * wv / KS, ge = G * (wv + 1) / KS;
  const int64_t wpr = K / 16;  // code words per row

  f32x4 acc_y[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc_y[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool xrow = li < B;
  const uint16_t* xp = x + (int64_t)li * K + 32 * q;

  // prefetch ring of code pairs and scales, PREFETCH groups deep
  u32x2 cbuf[kPrefetch][TILES];
  uint32_t sbuf[kPrefetch][TILES];
#pragma unroll
  for (int p = 0; p < kPrefetch; ++p) {
    const int64_t g = gb + p;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int64_t row = row0 + 16 * t;
      if (g < ge) {
        cbuf[p][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(codes + row * wpr + 8 * g + 2 * q));
        sbuf[p][t] = scales[row * G + g];
      } else {
        cbuf[p][t] = u32x2{0u, 0u};
        sbuf[p][t] = 0u;
      }
    }
  }
  u32x4 xa[4];
  auto load_x = [&](int64_t g, u32x4 (&dst)[4]) {
    if (xrow && g < ge) {
      const u32x4* s = reinterpret_cast<const u32x4*>(xp + 128 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = s[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  load_x(gb, xa);

  for (int64_t g0 = gb; g0 < ge; g0 += kPrefetch) {
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) {
      const int64_t g = g0 + p;
      if (g >= ge) break;
      u32x4 xn[4];
      load_x(g + 1, xn);
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mu = 0; mu < 4; ++mu) {
          const uint32_t w = cbuf[p][t][mu >> 1];
          const int fb = 4 * (mu & 1);
          u32x4 b;
#pragma unroll
          for (int d = 0; d < 4; ++d) b[d] = (w << (14 - 2 * (fb + d))) & 0xC000C000u;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[mu]), as_bf16x8(b), acc, 0, 0, 0);
        }
        const float s = f16_bits_to_f32(sbuf[p][t]) * 0.5f;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc_y[t][r] = __builtin_fmaf(s, acc[r], acc_y[t][r]);
        // refill this ring slot with group g + PREFETCH
        const int64_t gn = g + kPrefetch;
        if (gn < ge) {
          const int64_t row = row0 + 16 * t;
          cbuf[p][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(codes + row * wpr + 8 * gn + 2 * q));
          sbuf[p][t] = scales[row * G + gn];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = xn[i];
    }
  }

  // lane holds y[m = 4q + r][n = row0 + 16t]; reduce the KS partial sums
  if (KS > 1) {
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((wv * TILES + t) * 4 + r) * 64 + lane] = acc_y[t][r];
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = 0.f;
        for (int w = 0; w < KS; ++w) s += red[((w * TILES + t) * 4 + r) * 64 + lane];
        acc_y[t][r] = s;
      }
  }
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * q + r;
      if (m < B) y[(int64_t)m * N + row0 + 16 * t] = acc_y[t][r];
    }
}

}  // namespace

hipError_t launch_gemv_ternary(const uint16_t* x, int64_t B, const uint32_t* codes, const uint16_t* scales,
                               int64_t N, int64_t K, float* y, hipStream_t stream) {
  const int64_t G = K / kBlock;
  const int64_t tiles16 = N / 16;
  // Enough waves to cover the chip (256 CUs) several times over, and at least a
  // few groups per wave so the prefetch ring has work to overlap.
  int tiles = B > 4 ? 2 : 1;
  const int64_t wg = tiles16 / tiles;
  int ks = 1;
  while (ks < 8 && wg * ks < 2048 && G / (ks * 2) >= 2) ks *= 2;
  if (ks > G) ks = (int)G;
  const size_t lds = ks > 1 ? (size_t)ks * tiles * 4 * 64 * sizeof(float) : 0;
  const dim3 grid((unsigned)wg), block((unsigned)(64 * ks));
  if (tiles == 2)
    hipLaunchKernelGGL((gemv_ternary_kernel<2>), grid, block, lds, stream, x, (int)B, codes, scales, N, K, y, ks);
  else
    hipLaunchKernelGGL((gemv_ternary_kernel<1>), grid, block, lds, stream, x, (int)B, codes, scales, N, K, y, ks);
  return hipGetLastError();
}

}  // namespace tb
