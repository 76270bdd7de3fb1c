// Prefill GEMM with dense ternary weights, the decode contraction for M rows:
//   y[m][n] = sum_g f16(scale[n][g]) * sum_{k in g} t[n][k] * x[m][k]
//
// The one dense contraction of the path, so it runs on the matrix cores.  The
// group scale changes every 128 K, and applying it to fp32 partial sums would
// double the accumulator registers; instead each weight enters the MFMA as the
// fp16 value 2 t s, which is exact (s is fp16; doubling only moves the
// exponent), the activations enter as fp16 (bf16 -> fp16 is exact for
// 2^-14 <= |x| < 65504), and the fp32 accumulator runs over all of K.  The
// result is halved on the way out.
// Decode: a dense code word holds column c's field in nibble c % 8, bits 2-3
// for c < 8 and bits 0-1 for c >= 8.  Shifting the word left by 4, 6 and 2
// puts the fields of columns 2p, 8 + 2p and 9 + 2p at bits 6-7 of byte p (the
// field of column 2p + 1 is there already); one v_perm_b32 moves two such
// bytes to bytes 1 and 3 and the mask 0xC000C000 leaves the fp16 pair
// (2t, 2t') - bit 14 alone is the exponent of 2.0 in fp16.  One packed fp16
// multiply by (s, s) makes (2ts, 2t's).
// Tiling (first version): 128 x 128 output tile per workgroup of 4 waves, each
// wave 64 x 64 with v_mfma_f32_16x16x32_f16; K steps of 64 staged through LDS
// (fp16, double buffered, rows padded to spread banks).  Each K step reads the
// codes of 128 rows once (8 bytes per thread) and decodes them once for all
// 128 activation rows of the tile.
#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

constexpr int BM = 128, BN = 128, KT = 64;
constexpr int LDS_ROW = KT + 8;  // fp16 elements per LDS row (144 bytes)
constexpr int TILE_ELEMS = BM * LDS_ROW;

// fp16 pairs (2t, 2t') of the 16 columns of a dense code word, in column order.
__device__ __forceinline__ void decode_word_f16(uint32_t w, uint32_t (&out)[8]) {
  const uint32_t t4 = w << 4, t6 = w << 6, t2 = w << 2;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t sel = 0x0Cu | ((uint32_t)p << 8) | (0x0Cu << 16) | ((uint32_t)(4 + p) << 24);
    out[p] = __builtin_amdgcn_perm(w, t4, sel) & 0xC000C000u;       // columns 2p, 2p + 1
    out[4 + p] = __builtin_amdgcn_perm(t2, t6, sel) & 0xC000C000u;   // columns 8 + 2p, 9 + 2p
  }
}

__device__ __forceinline__ uint32_t bf16pair_to_f16pair(uint32_t w) {
  const float lo = bf16_to_f32(w & 0xffffu);
  const float hi = bf16_to_f32(w >> 16);
  return f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(256) gemm_ternary_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                           const uint32_t* __restrict__ codes,
                                                           const uint16_t* __restrict__ scales, int64_t N,
                                                           int64_t K, void* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][TILE_ELEMS];  // [stage][X | W][row][k]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = (wv >> 1) * 64, wn = (wv & 1) * 64;  // wave's sub-tile
  const int li = lane & 15, q = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t G = K / kBlock;
  const int nsteps = (int)(K / KT);

  // global -> register staging assignment
  // X: 128 rows x 64 k bf16 = 128 B per row; thread -> row tid/2, 32 k (64 B) at (tid&1)*32
  const int xr = tid >> 1, xk = (tid & 1) * 32;
  const bool xvalid = m0 + xr < M;
  const uint16_t* xsrc = x + (m0 + xr) * K + xk;
  // W: 128 rows x 64 k; thread -> row tid/2, the 32 columns of lane group
  // (k0 % 128) / 32 + (tid & 1) of the row's tile: two consecutive words
  const int wr = tid >> 1, wk = (tid & 1) * 32;
  const uint32_t* wsrc = codes + ((n0 + wr) >> 4) * G * 128 + 2 * (16 * (tid & 1) + ((n0 + wr) & 15));
  const uint16_t* ssrc = scales + (n0 + wr) * G;

  u32x4 xs[4];
  u32x2 cs;
  uint32_t ss;
  auto gload = [&](int step) {
    const int64_t k0 = (int64_t)step * KT;
    if (xvalid) {
      const u32x4* s = reinterpret_cast<const u32x4*>(xsrc + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[i] = s[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[i] = u32x4{0u, 0u, 0u, 0u};
    }
    cs = *reinterpret_cast<const u32x2*>(wsrc + (k0 / kBlock) * 128 + 64 * ((k0 % kBlock) / 64));
    ss = ssrc[k0 / kBlock];
  };
  auto lstore = [&](int stage) {
    // X: convert bf16 -> fp16 and store 32 elements of row xr
    uint16_t* xd = &lds[stage][0][xr * LDS_ROW + xk];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = bf16pair_to_f16pair(xs[i][j]);
      *reinterpret_cast<u32x4*>(xd + 8 * i) = o;
    }
    // W: decode 32 k of row wr into fp16 2*t*s, pairs (k, k+1)
    const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)ss);
    const f16x2 s2 = {sh, sh};
    uint16_t* wd = &lds[stage][1][wr * LDS_ROW + wk];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t bits[8];
      decode_word_f16(cs[j], bits);
      u32x4 o0, o1;
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const f16x2 v = __builtin_bit_cast(f16x2, bits[f]) * s2;
        if (f < 4) o0[f] = __builtin_bit_cast(uint32_t, v);
        else o1[f - 4] = __builtin_bit_cast(uint32_t, v);
      }
      *reinterpret_cast<u32x4*>(wd + 16 * j) = o0;
      *reinterpret_cast<u32x4*>(wd + 16 * j + 8) = o1;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    if (step + 1 < nsteps) gload(step + 1);
#pragma unroll
    for (int kk = 0; kk < KT; kk += 32) {
      f16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(&lds[cur][0][(wm + 16 * i + li) * LDS_ROW + kk + 8 * q]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(&lds[cur][1][(wn + 16 * j + li) * LDS_ROW + kk + 8 * q]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (step + 1 < nsteps) lstore(cur ^ 1);
    __syncthreads();
  }

  // lane holds acc[i][j][r] = 2 * y[m0 + wm + 16i + 4q + r][n0 + wn + 16j + li]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wm + 16 * i + 4 * q + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn + 16 * j + li;
        const float v = acc[i][j][r] * 0.5f;
        if constexpr (OUT_BF16)
          static_cast<uint16_t*>(y)[m * N + n] = (uint16_t)f32_to_bf16_rne(v);
        else
          static_cast<float*>(y)[m * N + n] = v;
      }
    }
}

}  // namespace

hipError_t launch_gemm_ternary(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                               int64_t N, int64_t K, void* y, int y_dtype, hipStream_t stream) {
  const int64_t mt = (M + BM - 1) / BM;
  if (mt > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(N / BN), (unsigned)mt), block(256);
  if (y_dtype == TB_BF16)
    hipLaunchKernelGGL((gemm_ternary_kernel<true>), grid, block, 0, stream, x, M, codes, scales, N, K, y);
  else
    hipLaunchKernelGGL((gemm_ternary_kernel<false>), grid, block, 0, stream, x, M, codes, scales, N, K, y);
  return hipGetLastError();
}

}  // namespace tb
