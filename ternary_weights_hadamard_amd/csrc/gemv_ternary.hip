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
// Work split: a workgroup owns 16 output rows; its KS waves split the K groups
// and reduce through LDS.  Latency: every wave keeps PREFETCH groups of codes
// and scales in flight, and the activations the workgroup needs are staged in
// LDS once (row stride padded by 16 bytes against bank conflicts) instead of
// being fetched from L2 group by group; when B*K is too large for LDS they are
// read from global memory two groups ahead.
#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

constexpr int kPrefetch = 8;
constexpr int kMaxXLdsBytes = 80 * 1024;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <bool XLDS>
__global__ void __launch_bounds__(512) gemv_ternary_kernel(const uint16_t* __restrict__ x, int B,
                                                            const uint32_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales, int64_t N,
                                                            int64_t K, float* __restrict__ y, int KS) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int li = lane & 15;  // batch row of the A operand / output row of the B operand
  const int q = lane >> 4;   // which 32-wide quarter of a group this lane covers
  const int64_t G = K / kBlock;
  const int64_t row = (int64_t)blockIdx.x * 16 + li;
  const int64_t gb = G * wv / KS, ge = G * (wv + 1) / KS;
  const uint32_t* cp = codes + row * (K / 16) + 2 * q;
  const uint16_t* sp = scales + row * G;

  // prefetch ring of code pairs and scales, PREFETCH groups deep, issued first
  u32x2 cbuf[kPrefetch];
  uint32_t sbuf[kPrefetch];
#pragma unroll
  for (int p = 0; p < kPrefetch; ++p) {
    const int64_t g = gb + p;
    if (g < ge) {
      cbuf[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(cp + 8 * g));
      sbuf[p] = sp[g];
    } else {
      cbuf[p] = u32x2{0u, 0u};
      sbuf[p] = 0u;
    }
  }

  const int64_t xstride = K + 8;  // LDS row stride in bf16 elements
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (XLDS ? (size_t)B * xstride * 2 : 0));
  if constexpr (XLDS) {
    // cooperative copy of x [B][K] into LDS, 16 bytes per lane
    const int64_t chunks = (int64_t)B * (K / 8);
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
      const int64_t b = c / (K / 8), kk = (c % (K / 8)) * 8;
      *reinterpret_cast<u32x4*>(xs + b * xstride + kk) = *reinterpret_cast<const u32x4*>(x + b * K + kk);
    }
    __syncthreads();
  }
  const bool xrow = li < B;
  auto load_x = [&](int64_t g, u32x4 (&dst)[4]) {
    if (xrow) {
      if constexpr (XLDS) {
        const u32x4* s = reinterpret_cast<const u32x4*>(xs + li * xstride + 128 * g + 32 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = s[i];
      } else {
        const u32x4* s = reinterpret_cast<const u32x4*>(x + (int64_t)li * K + 128 * g + 32 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = s[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x4 acc_y = {0.f, 0.f, 0.f, 0.f};
  u32x4 xa[4], xn[4];
  if (gb < ge) load_x(gb, xa);
  if (!XLDS && gb + 1 < ge) load_x(gb + 1, xn);

  for (int64_t g0 = gb; g0 < ge; g0 += kPrefetch) {
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) {
      const int64_t g = g0 + p;
      if (g >= ge) break;
      if constexpr (XLDS) {
        if (g + 1 < ge) load_x(g + 1, xn);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mu = 0; mu < 4; ++mu) {
        const uint32_t w = cbuf[p][mu >> 1];
        const int fb = 4 * (mu & 1);
        u32x4 bw;
#pragma unroll
        for (int d = 0; d < 4; ++d) bw[d] = (w << (14 - 2 * (fb + d))) & 0xC000C000u;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[mu]), as_bf16x8(bw), acc, 0, 0, 0);
      }
      const float s = f16_bits_to_f32(sbuf[p]) * 0.5f;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_y[r] = __builtin_fmaf(s, acc[r], acc_y[r]);
      // refill this ring slot with group g + PREFETCH
      const int64_t gn = g + kPrefetch;
      if (gn < ge) {
        cbuf[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(cp + 8 * gn));
        sbuf[p] = sp[gn];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = xn[i];
      if constexpr (!XLDS) {
        if (g + 2 < ge) load_x(g + 2, xn);
      }
    }
  }

  // lane holds y[m = 4q + r][n = row]; reduce the KS partial sums
  if (KS > 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wv * 4 + r) * 64 + lane] = acc_y[r];
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float s = 0.f;
      for (int w = 0; w < KS; ++w) s += red[(w * 4 + r) * 64 + lane];
      acc_y[r] = s;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * q + r;
    if (m < B) y[(int64_t)m * N + row] = acc_y[r];
  }
}

}  // namespace

hipError_t launch_gemv_ternary(const uint16_t* x, int64_t B, const uint32_t* codes, const uint16_t* scales,
                               int64_t N, int64_t K, float* y, hipStream_t stream) {
  const int64_t G = K / kBlock;
  const int64_t wg = N / 16;
  // Enough waves to cover the chip (256 CUs) several times over, while keeping
  // several groups per wave for the prefetch ring.
  int ks = 1;
  while (ks < 8 && wg * ks < 2048 && G / (ks * 2) >= 4) ks *= 2;
  const size_t xbytes = (size_t)B * (K + 8) * 2;
  const bool xlds = xbytes <= (size_t)kMaxXLdsBytes;
  const size_t lds = (xlds ? xbytes : 0) + (ks > 1 ? (size_t)ks * 4 * 64 * sizeof(float) : 0);
  const dim3 grid((unsigned)wg), block((unsigned)(64 * ks));
  if (xlds)
    hipLaunchKernelGGL((gemv_ternary_kernel<true>), grid, block, lds, stream, x, (int)B, codes, scales, N, K, y, ks);
  else
    hipLaunchKernelGGL((gemv_ternary_kernel<false>), grid, block, lds, stream, x, (int)B, codes, scales, N, K, y, ks);
  return hipGetLastError();
}

}  // namespace tb
