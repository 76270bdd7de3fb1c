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

constexpr int kPrefetch = 4;

template <int TILES>
__global__ void __launch_bounds__(512) gemv_ternary24_kernel(const uint16_t* __restrict__ x, int B,
                                                              const uint32_t* __restrict__ meta,
                                                              const uint32_t* __restrict__ signs,
                                                              const uint16_t* __restrict__ scales, int64_t N,
                                                              int64_t K, float* __restrict__ y, int KS) {
  extern __shared__ float red[];  // [KS][TILES][4][64]
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int li = lane & 15;
  const int q = lane >> 4;
  const int64_t G = K / kBlock;
  const int64_t nbase = (int64_t)blockIdx.x * (16 * TILES);
  const int64_t gb = G * wv / KS, ge = G * (wv + 1) / KS;
  const int64_t mpr = K / 32, spr = K / 64;  // meta / sign words per row
  const int sbit = 8 * (q & 1);              // first sign bit of this lane's quads in its sign word

  f32x4 acc_y[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc_y[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool xrow = li < B;
  const uint16_t* xp = x + (int64_t)li * K;
  // actual 8-wide K blocks of this lane's dense operand, for h = 0, 1: b0 + 2h and b0 + 2h + 8
  const int b0 = 4 * (q >> 1) + (q & 1);

  u32x2 mbuf[kPrefetch][TILES];  // (meta word, sign word) of row i
  uint32_t sbuf[kPrefetch][TILES][4];
  auto load_w = [&](int64_t g, u32x2& mw, uint32_t (&sc)[4], int t) {
    const int64_t row = nbase + 16 * t + li;
    mw[0] = __builtin_nontemporal_load(meta + row * mpr + 4 * g + q);
    mw[1] = __builtin_nontemporal_load(signs + row * spr + 2 * g + (q >> 1));
    const int64_t srow = nbase + 16 * t + 4 * q;
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = scales[(srow + r) * G + g];
  };
#pragma unroll
  for (int p = 0; p < kPrefetch; ++p)
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      if (gb + p < ge) {
        load_w(gb + p, mbuf[p][t], sbuf[p][t], t);
      } else {
        mbuf[p][t] = u32x2{0u, 0u};
        sbuf[p][t][0] = sbuf[p][t][1] = sbuf[p][t][2] = sbuf[p][t][3] = 0u;
      }
    }

  auto load_x = [&](int64_t g, u32x4 (&dst)[4]) {
    if (xrow && g < ge) {
      const uint16_t* base = xp + 128 * g;
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
  u32x4 xa[4];
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
        const uint32_t mw = mbuf[p][t][0];
        const uint32_t sw = mbuf[p][t][1];
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
        for (int r = 0; r < 4; ++r) acc_y[t][r] = __builtin_fmaf(f16_bits_to_f32(sbuf[p][t][r]), acc[r], acc_y[t][r]);
        if (g + kPrefetch < ge) load_w(g + kPrefetch, mbuf[p][t], sbuf[p][t], t);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = xn[i];
    }
  }

  // lane holds y[m = li][n = nbase + 16t + 4q + r]
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
  if (li < B) {
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      f32x4 o = acc_y[t];
      *reinterpret_cast<f32x4*>(y + (int64_t)li * N + nbase + 16 * t + 4 * q) = o;
    }
  }
}

}  // namespace

hipError_t launch_gemv_ternary24(const uint16_t* x, int64_t B, const uint32_t* meta, const uint32_t* signs,
                                 const uint16_t* scales, int64_t N, int64_t K, float* y, hipStream_t stream) {
  const int64_t G = K / kBlock;
  const int64_t tiles16 = N / 16;
  int tiles = B > 4 ? 2 : 1;
  const int64_t wg = tiles16 / tiles;
  int ks = 1;
  while (ks < 8 && wg * ks < 2048 && G / (ks * 2) >= 2) ks *= 2;
  if (ks > G) ks = (int)G;
  const size_t lds = ks > 1 ? (size_t)ks * tiles * 4 * 64 * sizeof(float) : 0;
  const dim3 grid((unsigned)wg), block((unsigned)(64 * ks));
  if (tiles == 2)
    hipLaunchKernelGGL((gemv_ternary24_kernel<2>), grid, block, lds, stream, x, (int)B, meta, signs, scales, N, K,
                       y, ks);
  else
    hipLaunchKernelGGL((gemv_ternary24_kernel<1>), grid, block, lds, stream, x, (int)B, meta, signs, scales, N, K,
                       y, ks);
  return hipGetLastError();
}

}  // namespace tb
