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
//
// The planes are tile-major (a 16-row tile and a 128-group together, row i's
// word w at position 16 w + i), so the operand words of a lane are where a
// whole-wave load puts them: meta word q of row i is lane (i, q)'s dword of
// the tile-group's 256 bytes.
// Staged path (batch <= 4): a wave owns one 16-row tile and a slice of at most
// CH groups of K.  It loads its slice of x first (staged through a private LDS
// area, then read in the operand layout), then per group one meta dword, one
// sign dword and one pair of scales straight into registers, all before the
// first product.  With the row-major planes this kernel started from, a
// slice was 16 short pieces per plane, staged through LDS (17408 x 5120:
// 10.8 us).  The K slices of a tile are the waves of one workgroup, added
// through LDS in a fixed order.
#include <algorithm>

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
  // tile-major planes: group g of this tile at tile-group nb G + g; meta word q
  // of row li at 16 q + li (the lane), sign word q / 2 at 16 (q / 2) + li,
  // the scales of rows 4q .. 4q+3 at 4q
  const int64_t nb = (int64_t)blockIdx.x;
  const uint32_t* mp = meta + nb * G * 64 + lane;
  const uint32_t* gp = signs + nb * G * 32 + (q >> 1) * 16 + li;
  const uint16_t* sp = scales + nb * G * 16 + 4 * q;

  u32x2 mbuf[kPrefetch];  // (meta word, sign word) of row li
  uint32_t sbuf[kPrefetch][4];
  auto load_w = [&](int64_t g, int p) {
    mbuf[p][0] = __builtin_nontemporal_load(mp + 64 * g);
    mbuf[p][1] = __builtin_nontemporal_load(gp + 32 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) sbuf[p][r] = sp[16 * g + r];
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

// bytes of one wave's activation staging area: x [B][CH][256 B]
__host__ __device__ constexpr int stage24_bytes(int ch, int b) { return b * ch * 256; }

template <int CH>
__global__ void __launch_bounds__(1024) gemv24_staged_kernel(const uint16_t* __restrict__ x, int B,
                                                             const uint32_t* __restrict__ meta,
                                                             const uint32_t* __restrict__ signs,
                                                             const uint16_t* __restrict__ scales, int64_t N,
                                                             int64_t K, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int KS = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, q = lane >> 4;
  const int64_t nb = blockIdx.x;
  const int G = (int)((uint64_t)K >> 7);
  // KS is a power of two (the launch doubles it): shifts, not divisions, so
  // that the wave reaches its first load sooner
  const int lg = __builtin_ctz((unsigned)KS);
  const int gb = (G * w) >> lg, ge = (G * (w + 1)) >> lg;
  const int n = ge - gb;  // 1 .. CH groups
  unsigned char* st_x = smem + (size_t)w * stage24_bytes(CH, B);  // [B][CH * 128] bf16
  float* red = reinterpret_cast<float*>(smem + (size_t)KS * stage24_bytes(CH, B));

  // 1. the x slice of each batch row first (every product needs it): 16
  //    chunks of 16 bytes per group
  constexpr int kXChunks = (16 * CH + 63) / 64;
  u32x4 x_st[4][kXChunks];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int t = 0; t < kXChunks; ++t) {
      const int c = lane + 64 * t;
      if (b < B && c < 16 * n) x_st[b][t] = *reinterpret_cast<const u32x4*>(x + (int64_t)b * K + 128 * gb + 8 * c);
    }
  // 2. each group's operand words straight from the tile-major planes, in
  //    group order (a product then waits only for its own group): meta word q
  //    of row li is the lane's dword of the tile-group's 256 bytes, sign word
  //    q / 2 of row li, and the scales of rows 4q .. 4q+3.  Slots past the
  //    slice repeat its last group.
  const int64_t tg0 = nb * G + gb;  // first tile-group of the slice
  uint32_t mw[CH], sw[CH];
  u32x2 sc[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int64_t tg = tg0 + min(j, n - 1);
    mw[j] = __builtin_nontemporal_load(meta + tg * 64 + lane);
    sw[j] = __builtin_nontemporal_load(signs + tg * 32 + (q >> 1) * 16 + li);
    sc[j] = *reinterpret_cast<const u32x2*>(scales + tg * 16 + 4 * q);
  }
  // 3. the x slice into this wave's LDS area (read back by the same wave only)
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int t = 0; t < kXChunks; ++t) {
      const int c = lane + 64 * t;
      if (b < B && c < 16 * n) *reinterpret_cast<u32x4*>(st_x + (b * CH * 128 + 8 * c) * 2) = x_st[b][t];
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // 4. the products.  Lanes of batch rows >= B read row B - 1 (their results
  // are never stored).
  const int sbit = 8 * (q & 1);
  const int b0 = 4 * (q >> 1) + (q & 1);
  const unsigned char* xrow = st_x + (size_t)min(li, B - 1) * CH * 128 * 2;
  f32x4 acc_y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int jj = min(j, n - 1);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 a;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int p_bit = sbit + 4 * h + d;
        a[d] = ((sw[j] << (15 - p_bit)) & 0x80008000u) | 0x3F803F80u;
      }
      const unsigned char* xb = xrow + jj * 256;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(xb + 16 * (b0 + 2 * h));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(xb + 16 * (b0 + 2 * h + 8));
      const u32x8 bx = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (h == 0)
        acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, bx),
                                                        acc, (int)mw[j], 0, 0);
      else
        acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, bx),
                                                        acc, (int)mw[j], 0, 1);
    }
    const uint32_t sv[4] = {sc[j][0] & 0xFFFFu, sc[j][0] >> 16, sc[j][1] & 0xFFFFu, sc[j][1] >> 16};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = __builtin_fmaf(f16_bits_to_f32(sv[r]), acc[r], acc_y[r]);
      acc_y[r] = j < n ? v : acc_y[r];
    }
  }

  // 5. lane holds y[b = li][n = 16 nb + 4q + r]; slices added in order
  if (KS > 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(w * 4 + r) * 64 + lane] = acc_y[r];
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      for (int u = 1; u < KS; ++u) acc_y[r] += red[(u * 4 + r) * 64 + lane];
  }
  if (li < B) *reinterpret_cast<f32x4*>(y + (int64_t)li * N + 16 * nb + 4 * q) = acc_y;
}

}  // namespace

hipError_t launch_gemv_ternary24(const uint16_t* x, int64_t B, const uint32_t* meta, const uint32_t* signs,
                                 const uint16_t* scales, int64_t N, int64_t K, float* y, hipStream_t stream) {
  const int64_t G = K / kBlock;
  const int64_t wg = N / 16;
  {
    // staged path: the fewest K slices (a power of two, at most 16) that leave
    // at most 5 groups per slice, or 9 when 16 slices are not enough.  Per
    // launch, batch 1 (graph-replayed): 17408 x 5120 10.8 us with 8 slices of
    // 5 groups (11.0 with 4 of 10); 5120 x 5120 6.2 us with 8 (8.4 with 16);
    // 5120 x 17408 17.7 us with 16 slices of 9 groups, which need 113 KB of
    // LDS (38.2 us on the unstaged kernel the former 96 KB limit left it to).
    int ks = 1;
    // (every slice keeps at least one group: 2 ks <= G before doubling)
    while (ks < 16 && 2 * ks <= G && (G + ks - 1) / ks > 5) ks *= 2;
    const int64_t ch = (G + ks - 1) / ks;
    if (B <= 4 && ch <= 9) {
      const int CH = ch <= 5 ? 5 : 9;
      const size_t lds = (size_t)ks * stage24_bytes(CH, (int)B) + (size_t)ks * 4 * 64 * sizeof(float);
      if (lds <= 128 * 1024) {
        const dim3 grid((unsigned)wg), block((unsigned)(64 * ks));
        if (CH == 5)
          hipLaunchKernelGGL((gemv24_staged_kernel<5>), grid, block, lds, stream, x, (int)B, meta, signs, scales, N,
                             K, y);
        else
          hipLaunchKernelGGL((gemv24_staged_kernel<9>), grid, block, lds, stream, x, (int)B, meta, signs, scales, N,
                             K, y);
        return hipGetLastError();
      }
    }
  }
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
