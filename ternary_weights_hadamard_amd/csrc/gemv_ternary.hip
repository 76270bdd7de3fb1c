// Decode GEMV with dense ternary weights:
//   y[b][n] = sum_g f16(scale[n][g]) * sum_{k in g} t[n][k] * x[b][k]
// (mhpq.cn/news/1159370 §4.2: read the weight bits, expand, scale, multiply).
//
// HBM bound: every weight is streamed once at 2 bits plus 1/8 bit of scale,
// so the kernel is built to spend as little vector-ALU work per weight as
// possible and to keep many code loads in flight.
//   * The contraction runs on v_mfma_scale_f32_16x16x128_f8f6f4: the weights
//     are its fp4 operand (one 16-row x 128-column tile per instruction), the
//     activations its e4m3 operand with E8M0 block scales (act8.h: each bf16
//     activation is the exact sum of four e4m3 sub-row values).
//   * A tile word holds 16 two-bit fields laid out so that (w & 0xCCCCCCCC) and
//     ((w << 2) & 0xCCCCCCCC) are eight fp4 values each: bit 3 of a nibble is
//     the sign, bit 2 the exponent bit of 2.0, so +1 -> 2.0, -1 -> -2.0, 0 -> 0.
//     Three VALU operations expand 16 weights.
//   * Lane (i, q) holds output rows 4q .. 4q + 3 of column i: the four sub-rows
//     of batch row 4m + q.  Their sum times f16(scale) / 2 is the group's
//     contribution.
// Work split: a wave owns one 16-row tile and a contiguous range of groups;
// four waves per workgroup cover 4 / KS tiles x KS group ranges, and split
// ranges are added through LDS.  Each wave keeps kPrefetch groups of codes and
// scales in flight and loads the activation operand two groups ahead (it is
// read by every wave and stays in cache).
#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kPrefetch = 8;
constexpr int kWaves = 4;

template <int NB4>
struct ActFrag {
  i32x8 v[NB4];
  int s[NB4];
};

template <int NB4>
__global__ void __launch_bounds__(256) gemv_ternary_kernel(const uint8_t* __restrict__ act, int B,
                                                            const uint32_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales, int64_t N,
                                                            int64_t K, float* __restrict__ y, int KS) {
  __shared__ float red[kWaves][NB4][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, q = lane >> 4;
  const int ks = wv % KS;
  const int64_t nb = (int64_t)blockIdx.x * (kWaves / KS) + wv / KS;
  const bool live = nb < N / 16;
  const int G = (int)(K / kBlock);
  const int gb = G * ks / KS, ge = G * (ks + 1) / KS;

  float acc[NB4];
#pragma unroll
  for (int m = 0; m < NB4; ++m) acc[m] = 0.f;

  if (live && gb < ge) {
    const uint32_t* cp = codes + (size_t)nb * G * 128 + 2 * lane;
    const uint16_t* sp = scales + (size_t)(16 * nb + i) * G;
    // activation operand rows of this lane: batch 4m + i/4, sub-row i % 4
    const uint8_t* av_base[NB4];
    const uint8_t* as_base[NB4];
    bool arow[NB4];
#pragma unroll
    for (int m = 0; m < NB4; ++m) {
      const int b = 4 * m + (i >> 2);
      arow[m] = b < B;
      const size_t row = (size_t)(arow[m] ? b : 0) * G;
      av_base[m] = act + (row * 16 + (i & 3) * 4 + q) * 32;
      as_base[m] = act + (size_t)4 * B * K + row * 16 + (i & 3) * 4 + q;
    }
    auto load_act = [&](int g, ActFrag<NB4>& f) {
#pragma unroll
      for (int m = 0; m < NB4; ++m) {
        if (arow[m]) {
          const u32x4* p = reinterpret_cast<const u32x4*>(av_base[m] + (size_t)g * 512);
          const u32x4 lo = p[0], hi = p[1];
          f.v[m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          f.s[m] = as_base[m][(size_t)g * 16];
        } else {
          f.v[m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
          f.s[m] = 127;
        }
      }
    };

    u32x2 cr[kPrefetch];
    uint32_t sr[kPrefetch];
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) {
      const int g = min(gb + p, ge - 1);
      cr[p] = *reinterpret_cast<const u32x2*>(cp + (size_t)g * 128);
      sr[p] = sp[g];
    }
    ActFrag<NB4> fa[2];
    load_act(gb, fa[0]);
    load_act(min(gb + 1, ge - 1), fa[1]);

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int g0 = gb; g0 < ge; g0 += kPrefetch) {
#pragma unroll
      for (int p = 0; p < kPrefetch; ++p) {
        const int g = g0 + p;
        if (g >= ge) break;
        ActFrag<NB4>& f = fa[p & 1];
        const uint32_t w0 = cr[p][0], w1 = cr[p][1];
        const i32x4 bw = {(int)(w0 & 0xCCCCCCCCu), (int)((w0 << 2) & 0xCCCCCCCCu), (int)(w1 & 0xCCCCCCCCu),
                          (int)((w1 << 2) & 0xCCCCCCCCu)};
        const i32x8 b8 = {bw[0], bw[1], bw[2], bw[3], 0, 0, 0, 0};
        const float s = f16_bits_to_f32(sr[p]) * 0.5f;
#pragma unroll
        for (int m = 0; m < NB4; ++m) {
          const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.v[m], b8, zero, 0, 4, 0, f.s[m], 0, 127);
          acc[m] = __builtin_fmaf(s, (d[0] + d[1]) + (d[2] + d[3]), acc[m]);
        }
        // refill: codes kPrefetch groups ahead, activations two ahead (clamped to the range)
        const int gn = min(g + kPrefetch, ge - 1);
        cr[p] = *reinterpret_cast<const u32x2*>(cp + (size_t)gn * 128);
        sr[p] = sp[gn];
        load_act(min(g + 2, ge - 1), f);
      }
    }
  }

  if (KS > 1) {
#pragma unroll
    for (int m = 0; m < NB4; ++m) red[wv][m][lane] = acc[m];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int m = 0; m < NB4; ++m)
      for (int w = 1; w < KS; ++w) acc[m] += red[wv + w][m][lane];
  }
  if (!live) return;
#pragma unroll
  for (int m = 0; m < NB4; ++m) {
    const int b = 4 * m + q;
    if (b < B) y[(size_t)b * N + 16 * nb + i] = acc[m];
  }
}

}  // namespace

hipError_t launch_gemv_ternary(const uint8_t* act, int64_t B, const uint32_t* codes, const uint16_t* scales,
                               int64_t N, int64_t K, float* y, hipStream_t stream) {
  const int64_t tiles = N / 16, G = K / kBlock;
  // split K over up to 4 waves while the tiles alone give fewer than 2048
  // waves, keeping at least 4 groups per wave
  int ks = 1;
  while (ks < kWaves && tiles * ks < 2048 && G >= 8 * ks) ks *= 2;
  const int64_t per_block = kWaves / ks;
  const dim3 grid((unsigned)((tiles + per_block - 1) / per_block)), block(64 * kWaves);
  const int nb4 = (int)((B + 3) / 4);
  switch (nb4) {
    case 1: hipLaunchKernelGGL(gemv_ternary_kernel<1>, grid, block, 0, stream, act, (int)B, codes, scales, N, K, y, ks); break;
    case 2: hipLaunchKernelGGL(gemv_ternary_kernel<2>, grid, block, 0, stream, act, (int)B, codes, scales, N, K, y, ks); break;
    case 3: hipLaunchKernelGGL(gemv_ternary_kernel<3>, grid, block, 0, stream, act, (int)B, codes, scales, N, K, y, ks); break;
    default: hipLaunchKernelGGL(gemv_ternary_kernel<4>, grid, block, 0, stream, act, (int)B, codes, scales, N, K, y, ks); break;
  }
  return hipGetLastError();
}

}  // namespace tb
