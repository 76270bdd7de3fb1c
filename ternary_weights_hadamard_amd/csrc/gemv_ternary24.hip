// Decode GEMV with 2:4 ternary weights (mhpq.cn/news/1159370 §1.2: two of
// every four kept, each kept element +-1 times the group scale):
//   y[b][n] = sum_g f16(scale[n][g]) * sum_q (+-x[b][4q + idx0] +- x[b][4q + idx1])
//
// gfx950's sparse matrix instruction v_smfmac_f32_16x16x64_bf16 takes a 16x64
// operand stored as 16x32 kept values plus a 2-bit position per kept value,
// two per quad, the first in the low bits: exactly the meta nibble of this
// format.  So the meta words go to the instruction untouched (the two 16-bit
// halves of one word are the two SMFMACs of a 128-group, picked by ABID), and
// the kept values are bf16 +-1 made from the sign plane with one shift and one
// and-or per pair: the sign bits of a quad's two kept elements sit 16 bits
// apart, like the sign bits of a bf16 pair.
// Operand placement (from the instruction's layout): lane (i, q) supplies the
// kept values of row i for 16 consecutive sparse K and the dense x values of
// batch row i at two 8-wide K blocks; D[4q + r][i] returns in lane (i, q).
// The 64-wide windows are mapped to actual K so that lane q of SMFMAC h covers
// K 128g + 32q + 16h .. +15: one meta word and one sign word per lane and group.
#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

constexpr int kPrefetch = 8;
constexpr int kMaxXLdsBytes = 80 * 1024;

template <bool XLDS>
__global__ void __launch_bounds__(512) gemv_ternary24_kernel(const uint16_t* __restrict__ x, int B,
                                                              const uint32_t* __restrict__ meta,
                                                              const uint32_t* __restrict__ signs,
                                                              const uint16_t* __restrict__ scales, int64_t N,
                                                              int64_t K, float* __restrict__ y, int KS) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int li = lane & 15;
  const int q = lane >> 4;
  const int64_t G = K / kBlock;
  const int64_t nbase = (int64_t)blockIdx.x * 16;
  const int64_t gb = G * wv / KS, ge = G * (wv + 1) / KS;
  const int sbit = 8 * (q & 1);  // first sign bit of this lane's quads in its sign word
  const uint32_t* mp = meta + (nbase + li) * (K / 32) + q;
  const uint32_t* gp = signs + (nbase + li) * (K / 64) + (q >> 1);
  const uint16_t* sp = scales + (nbase + 4 * q) * G;  // rows 4q .. 4q+3 of the tile

  u32x2 mbuf[kPrefetch];  // (meta word, sign word) of row li
  uint32_t sbuf[kPrefetch][4];
  auto load_w = [&](int64_t g, int p) {
    mbuf[p][0] = __builtin_nontemporal_load(mp + 4 * g);
    mbuf[p][1] = __builtin_nontemporal_load(gp + 2 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) sbuf[p][r] = sp[r * G + g];
  };
#pragma unroll
  for (int p = 0; p < kPrefetch; ++p) {
    if (gb + p < ge) {
      load_w(gb + p, p);
    } else {
      mbuf[p] = u32x2{0u, 0u};
      sbuf[p][0] = sbuf[p][1] = sbuf[p][2] = sbuf[p][3] = 0u;
    }
  }

  const int64_t xstride = K + 8;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (XLDS ? (size_t)B * xstride * 2 : 0));
  if constexpr (XLDS) {
    const int64_t chunks = (int64_t)B * (K / 8);
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
      const int64_t b = c / (K / 8), kk = (c % (K / 8)) * 8;
      *reinterpret_cast<u32x4*>(xs + b * xstride + kk) = *reinterpret_cast<const u32x4*>(x + b * K + kk);
    }
    __syncthreads();
  }
  // actual 8-wide K blocks of this lane's dense operand, for h = 0, 1: b0 + 2h and b0 + 2h + 8
  const int b0 = 4 * (q >> 1) + (q & 1);
  const bool xrow = li < B;
  auto load_x = [&](int64_t g, u32x4 (&dst)[4]) {
    if (xrow) {
      const uint16_t* base = XLDS ? xs + li * xstride + 128 * g : x + (int64_t)li * K + 128 * g;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        dst[2 * h] = *reinterpret_cast<const u32x4*>(base + 8 * (b0 + 2 * h));
        dst[2 * h + 1] = *reinterpret_cast<const u32x4*>(base + 8 * (b0 + 2 * h + 8));
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
      const uint32_t mw = mbuf[p][0];
      const uint32_t sw = mbuf[p][1];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 a;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int p_bit = sbit + 4 * h + d;
          a[d] = ((sw << (15 - p_bit)) & 0x80008000u) | 0x3F803F80u;
        }
        u32x8 bx;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bx[i] = xa[2 * h][i];
          bx[4 + i] = xa[2 * h + 1][i];
        }
        if (h == 0)
          acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x16, bx), acc, (int)mw, 0, 0);
        else
          acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x16, bx), acc, (int)mw, 0, 1);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_y[r] = __builtin_fmaf(f16_bits_to_f32(sbuf[p][r]), acc[r], acc_y[r]);
      if (g + kPrefetch < ge) load_w(g + kPrefetch, p);
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = xn[i];
      if constexpr (!XLDS) {
        if (g + 2 < ge) load_x(g + 2, xn);
      }
    }
  }

  // lane holds y[m = li][n = nbase + 4q + r]
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
  if (li < B) *reinterpret_cast<f32x4*>(y + (int64_t)li * N + nbase + 4 * q) = acc_y;
}

}  // namespace

hipError_t launch_gemv_ternary24(const uint16_t* x, int64_t B, const uint32_t* meta, const uint32_t* signs,
                                 const uint16_t* scales, int64_t N, int64_t K, float* y, hipStream_t stream) {
  const int64_t G = K / kBlock;
  const int64_t wg = N / 16;
  int ks = 1;
  while (ks < 8 && wg * ks < 2048 && G / (ks * 2) >= 4) ks *= 2;
  const size_t xbytes = (size_t)B * (K + 8) * 2;
  const bool xlds = xbytes <= (size_t)kMaxXLdsBytes;
  const size_t lds = (xlds ? xbytes : 0) + (ks > 1 ? (size_t)ks * 4 * 64 * sizeof(float) : 0);
  const dim3 grid((unsigned)wg), block((unsigned)(64 * ks));
  if (xlds)
    hipLaunchKernelGGL((gemv_ternary24_kernel<true>), grid, block, lds, stream, x, (int)B, meta, signs, scales, N, K,
                       y, ks);
  else
    hipLaunchKernelGGL((gemv_ternary24_kernel<false>), grid, block, lds, stream, x, (int)B, meta, signs, scales, N,
                       K, y, ks);
  return hipGetLastError();
}

}  // namespace tb
