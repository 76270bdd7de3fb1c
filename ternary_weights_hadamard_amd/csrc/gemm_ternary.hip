// Prefill GEMM with dense ternary weights, the decode contraction for M rows:
//   y[m][n] = sum_g f16(scale[n][g]) * sum_{k in g} t[n][k] * x[m][k]
//
// The one dense contraction of the path, so it runs on the matrix cores, with
// bf16 operands: the activations go to LDS as they are (no conversion) and
// each weight enters as the bf16 value 2t (exact).  A 128-K group's products
// accumulate in fp32 registers of their own; at the end of the group they are
// added to the result accumulators times the group's fp16 scale (one FMA per
// accumulator, the scale taken straight from fp16).  The result is halved on
// the way out.
// Decode: a dense code word holds column c's field in nibble c % 8, bits 2-3
// for c < 8 and bits 0-1 for c >= 8.  Shifting the word left by 4, 6 and 2
// puts the fields of columns 2p, 8 + 2p and 9 + 2p at bits 6-7 of byte p (the
// field of column 2p + 1 is there already); one v_perm_b32 moves two such
// bytes to bytes 1 and 3 and the mask 0xC000C000 leaves the bf16 pair
// (2t, 2t') - bit 14 alone is the exponent of 2.0.
// Tiling: 128 x 128 output tile per workgroup of 4 waves, each wave 64 x 64
// with v_mfma_f32_16x16x32_bf16; K steps of 64 staged through LDS (double
// buffered), two steps per scale group.  An LDS row is 128 bytes, eight
// 16-byte chunks; chunk c of row r is stored at c ^ F(r), F(r) = (r ^ (((r >> 2)
// ^ (r >> 3)) & 1)) & 7.  With it the matrix-operand reads (16 lanes read one
// chunk of 16 consecutive rows) and the tile writes (16 lanes write chunks i
// and 4 + i of 8 consecutive rows) touch distinct banks, whether the LDS
// serves 8 lanes from 32 banks or 16 lanes from 64 (checked by enumeration);
// against padded 144-byte rows it is about 2 % faster and 10 KB smaller.
// Each K
// step reads the codes of 128 rows once (8 bytes per thread) and decodes them
// once for all 128 activation rows of the tile.
// Rotated output (ROT): the output tile is 128 columns wide, one 128-block of
// N, so the back-rotation y = R_N y' (the second transform of
// dpshk.com/news/5289456 §4.2, fused with the product) runs in the epilogue:
// the tile goes to LDS in fp32, each 16-lane group transforms a row with the
// in-register butterflies of the activation transform, and the result is
// rounded once.
// At most 16 rows of activations take the kernel of gemm_skinny.hip instead
// (unrotated output; rotated output keeps the path below).
// Split K (few rows of activations, so few output tiles): workgroup z of S
// takes the scale groups [G z / S, G (z + 1) / S) and writes its fp32 partial
// result to a caller-provided workspace; a second kernel adds the S partials
// in order (the result does not depend on timing) and converts.
#include <algorithm>

#include "fwht_lanes.h"
#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

constexpr int BM = 128, BN = 128, KT = 64;
constexpr int LDS_ROW = KT;  // bf16 elements per LDS row (128 bytes, chunks swizzled)
constexpr int kWRing = 2;        // groups of codes and scales in flight ahead
constexpr int TILE_ELEMS = BM * LDS_ROW;
constexpr int TROW = BN + 4;  // fp32 elements per row of the rotation epilogue's tile
// LDS of the main loop ([stage][X | W][row][k], 64 KB) or of the epilogue tile
constexpr int kLdsElems = 2 * 2 * TILE_ELEMS > BM * TROW * 2 ? 2 * 2 * TILE_ELEMS : BM * TROW * 2;

// element offset of (row r, element k) in a swizzled LDS tile
__device__ __forceinline__ int lds_off(int r, int k) {
  const int f = (r ^ (((r >> 2) ^ (r >> 3)) & 1)) & 7;
  return r * LDS_ROW + ((((k >> 3) ^ f) & 7) << 3) + (k & 7);
}

// bf16 pairs (2t, 2t') of the 16 columns of a dense code word, in column order.
__device__ __forceinline__ void decode_word_bf16(uint32_t w, uint32_t (&out)[8]) {
  const uint32_t t4 = w << 4, t6 = w << 6, t2 = w << 2;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t sel = 0x0Cu | ((uint32_t)p << 8) | (0x0Cu << 16) | ((uint32_t)(4 + p) << 24);
    out[p] = __builtin_amdgcn_perm(w, t4, sel) & 0xC000C000u;       // columns 2p, 2p + 1
    out[4 + p] = __builtin_amdgcn_perm(t2, t6, sel) & 0xC000C000u;   // columns 8 + 2p, 9 + 2p
  }
}

template <bool OUT_BF16, bool ROT>
__global__ void __launch_bounds__(256, 2) gemm_ternary_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                           const uint32_t* __restrict__ codes,
                                                           const uint16_t* __restrict__ scales, int64_t N,
                                                           int64_t K, void* __restrict__ y, int splits) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_mem[kLdsElems];
  uint16_t(*lds)[2][TILE_ELEMS] = reinterpret_cast<uint16_t(*)[2][TILE_ELEMS]>(lds_mem);  // [stage][X | W]
  __shared__ uint16_t lds_s[2][BN];                                         // [stage][weight row] fp16 scale
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = (wv >> 1) * 64, wn = (wv & 1) * 64;  // wave's sub-tile
  const int li = lane & 15, q = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t G = K / kBlock;
  // this workgroup's scale groups [gb, ge); output: y, or partial z of the workspace
  const int64_t gb = G * blockIdx.z / splits, ge = G * (blockIdx.z + 1) / splits;

  // global -> register staging assignment
  // X: 128 rows x 64 k bf16 = 128 B per row; thread -> row tid/2, 32 k (64 B) at (tid&1)*32
  // rows past M read row M - 1 instead: an activation row reaches only its own
  // output row, and those are never stored
  const int xr = tid >> 1, xk = (tid & 1) * 32;
  const uint16_t* xsrc = x + std::min<int64_t>(m0 + xr, M - 1) * K + gb * kBlock + xk;
  // W: 128 rows x 64 k; thread -> row tid/2, the 32 columns of lane group
  // (k0 % 128) / 32 + (tid & 1) of the row's tile: two consecutive words
  const int wr = tid >> 1, wk = (tid & 1) * 32;
  const uint32_t* wsrc = codes + ((n0 + wr) >> 4) * G * 128 + gb * 128 + 2 * (16 * (tid & 1) + ((n0 + wr) & 15));
  // scales [N/16][G][16]: row n's scale of group g at ((n / 16) G + g) 16 + n % 16
  const uint16_t* ssrc = scales + ((n0 + wr) >> 4) * G * 16 + gb * 16 + ((n0 + wr) & 15);

  // Activations come two K steps ahead through two register sets, one per
  // step parity (from L2: every column tile reads them; one step of products
  // is shorter than an L2 round trip).  The codes and scales, read once from
  // HBM, come kWRing groups ahead through a ring of registers, so their
  // latency is hidden behind several steps of work rather than one.  Every
  // prefetch is issued, clamped to the last step or group past the range, so
  // the wait counts are the same on every path.
  u32x4 xs[2][4];       // [step parity]
  u32x2 cw[kWRing][2];  // [ring slot][step of the group]
  uint32_t sw[kWRing];
  const int nsteps = 2 * (int)(ge - gb);
  auto gload_x = [&](int step) {
    const int64_t k0 = (int64_t)std::min(step, nsteps - 1) * KT;
    const u32x4* s = reinterpret_cast<const u32x4*>(xsrc + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[step & 1][i] = s[i];
  };
  // codes and scale of group gi (relative to gb) into ring slot `slot`; groups
  // past the range reload the last one (never used)
  auto gload_w = [&](int gi, int slot) {
    const int64_t g = std::min<int64_t>(gi, ge - gb - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) cw[slot][h] = *reinterpret_cast<const u32x2*>(wsrc + g * 128 + 64 * h);
    sw[slot] = ssrc[g * 16];
  };
  // the step in registers whose parity is `stage` into LDS stage `stage`
  auto lstore = [&](int stage, int slot, int h) {
    // X: 32 bf16 of row xr, as they are
    uint16_t* xd = lds[stage][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(xd + lds_off(xr, xk + 8 * i)) = xs[stage][i];
    // W: decode 32 k of row wr into bf16 2t, pairs (k, k+1)
    uint16_t* wd = lds[stage][1];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t bits[8];
      decode_word_bf16(cw[slot][h][j], bits);
      *reinterpret_cast<u32x4*>(wd + lds_off(wr, wk + 16 * j)) = u32x4{bits[0], bits[1], bits[2], bits[3]};
      *reinterpret_cast<u32x4*>(wd + lds_off(wr, wk + 16 * j + 8)) = u32x4{bits[4], bits[5], bits[6], bits[7]};
    }
    if ((tid & 1) == 0) lds_s[stage][wr] = (uint16_t)sw[slot];
  };

  // acc: the result; accg: the current scale group's products
  f32x4 acc[4][4], accg[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // the MFMAs of one K step from LDS stage `st`; FIRST starts the group
  auto mfma_step = [&](int st, bool first) {
#pragma unroll
    for (int kk = 0; kk < KT; kk += 32) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&lds[st][0][lds_off(wm + 16 * i + li, kk + 8 * q)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&lds[st][1][lds_off(wn + 16 * j + li, kk + 8 * q)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          accg[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], (first && kk == 0) ? zero : accg[i][j], 0,
                                                                 0, 0);
    }
  };

  // one scale group: its two K steps from LDS stages 0 and 1; the group's
  // codes are in ring slot `slot`, the next group's in slot `slot` + 1
  const int ngroups = (int)(ge - gb);
  auto group = [&](int gi, int slot) {
    // first step of the group from stage 0; step 2 gi + 1 goes to stage 1
    // and its registers refill with step 2 gi + 3
    mfma_step(0, true);
    lstore(1, slot, 1);
    gload_x(2 * gi + 3);
    // the group's codes are all in LDS now: refill its slot kWRing groups ahead
    gload_w(gi + kWRing, slot);
    __syncthreads();
    // second step from stage 1; step 2 gi + 2 goes to stage 0 and its
    // registers refill with step 2 gi + 4
    const bool more = gi + 1 < ngroups;
    mfma_step(1, false);
    // fold the group: lane's column n = n0 + wn + 16 j + li
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = (float)__builtin_bit_cast(_Float16, lds_s[1][wn + 16 * j + li]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(accg[i][j][r], sc, acc[i][j][r]);
    }
    if (more) lstore(0, (slot + 1) % kWRing, 0);
    gload_x(2 * gi + 4);
    __syncthreads();
  };

#pragma unroll
  for (int r = 0; r < kWRing; ++r) gload_w(r, r);
  gload_x(0);
  lstore(0, 0, 0);
  gload_x(1);
  gload_x(2);
  __syncthreads();
  for (int gi = 0; gi < ngroups; gi += kWRing) {
#pragma unroll
    for (int r = 0; r < kWRing; ++r)
      if (gi + r < ngroups) group(gi + r, r);
  }

  // lane holds acc[i][j][r] = 2 * y[m0 + wm + 16i + 4q + r][n0 + wn + 16j + li]
  if constexpr (ROT) {
    // the tile in fp32, rows padded (the main loop's last barrier has passed)
    static_assert(BM * TROW * sizeof(float) <= sizeof(lds_mem), "rotation tile exceeds LDS");
    float* t = reinterpret_cast<float*>(lds_mem);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) t[(wm + 16 * i + 4 * q + r) * TROW + wn + 16 * j + li] = acc[i][j][r] * 0.5f;
    __syncthreads();
    const int sub = tid & 15;
    for (int row = tid >> 4; row < BM; row += 16) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(t + row * TROW + 8 * sub);
      const f32x4 b = *reinterpret_cast<const f32x4*>(t + row * TROW + 8 * sub + 4);
      float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      fwht128_lanes(v, sub);
      const int64_t m = m0 + row;
      if (m >= M) continue;
      const int64_t base = m * N + n0 + 8 * sub;
      if constexpr (OUT_BF16) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = f32_to_bf16_rne(v[2 * e] * kInvSqrt128) | (f32_to_bf16_rne(v[2 * e + 1] * kInvSqrt128) << 16);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + base) = w;
      } else {
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = v[e] * kInvSqrt128;
          hi[e] = v[4 + e] * kInvSqrt128;
        }
        *reinterpret_cast<f32x4*>(static_cast<float*>(y) + base) = lo;
        *reinterpret_cast<f32x4*>(static_cast<float*>(y) + base + 4) = hi;
      }
    }
    return;
  }
  if (splits > 1) y = static_cast<float*>(y) + (size_t)blockIdx.z * M * N;
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

// y = sum over s < S of part[s] (in order), rounded to bf16 or kept fp32;
// MN is a multiple of 4.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, int S, int64_t MN,
                                                            void* __restrict__ y) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; e < MN; e += stride) {
    f32x4 a = *reinterpret_cast<const f32x4*>(part + e);
    for (int s = 1; s < S; ++s) {
      const f32x4 b = *reinterpret_cast<const f32x4*>(part + (size_t)s * MN + e);
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] += b[r];
    }
    if constexpr (OUT_BF16) {
      const uint32_t lo = f32_to_bf16_rne(a[0]) | (f32_to_bf16_rne(a[1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(a[2]) | (f32_to_bf16_rne(a[3]) << 16);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + e) = u32x2{lo, hi};
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(y) + e) = a;
    }
  }
}

// The S partials summed in order, then each 128-block of a row rotated back
// (R_N) by one 16-lane group, rounded once.  MN is a multiple of 128.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) splitk_reduce_rot_kernel(const float* __restrict__ part, int S, int64_t MN,
                                                                void* __restrict__ y) {
  const int sub = threadIdx.x & 15;
  const int64_t nblk = MN / kBlock, stride = (int64_t)gridDim.x * 16;
  for (int64_t bk = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4); bk - (threadIdx.x >> 4) < nblk; bk += stride) {
    // every lane of the wave runs the cross-lane rounds; lanes past the end carry zeros
    const bool live = bk < nblk;
    const int64_t e = (live ? bk : 0) * kBlock + 8 * sub;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      a = *reinterpret_cast<const f32x4*>(part + e);
      b = *reinterpret_cast<const f32x4*>(part + e + 4);
      for (int s = 1; s < S; ++s) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(part + (size_t)s * MN + e);
        const f32x4 d = *reinterpret_cast<const f32x4*>(part + (size_t)s * MN + e + 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] += c[r];
          b[r] += d[r];
        }
      }
    }
    float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    fwht128_lanes(v, sub);
    if (!live) continue;
    if constexpr (OUT_BF16) {
      u32x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        w[r] = f32_to_bf16_rne(v[2 * r] * kInvSqrt128) | (f32_to_bf16_rne(v[2 * r + 1] * kInvSqrt128) << 16);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + e) = w;
    } else {
      f32x4 lo, hi;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lo[r] = v[r] * kInvSqrt128;
        hi[r] = v[4 + r] * kInvSqrt128;
      }
      *reinterpret_cast<f32x4*>(static_cast<float*>(y) + e) = lo;
      *reinterpret_cast<f32x4*>(static_cast<float*>(y) + e + 4) = hi;
    }
  }
}

hipError_t launch_gemm(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales, int64_t N,
                       int64_t K, void* y, bool bf16_out, bool rot, int splits, hipStream_t stream) {
  const int64_t mt = (M + BM - 1) / BM;
  if (mt > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(N / BN), (unsigned)mt, (unsigned)splits), block(256);
#define TB_GEMM(B_, R_) \
  hipLaunchKernelGGL((gemm_ternary_kernel<B_, R_>), grid, block, 0, stream, x, M, codes, scales, N, K, y, splits)
  if (rot) {
    if (bf16_out)
      TB_GEMM(true, true);
    else
      TB_GEMM(false, true);
  } else {
    if (bf16_out)
      TB_GEMM(true, false);
    else
      TB_GEMM(false, false);
  }
#undef TB_GEMM
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_ternary(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                               int64_t N, int64_t K, void* y, int y_dtype, hipStream_t stream) {
  if (M <= kSkinnyMaxRows) return launch_gemm_skinny(x, M, codes, scales, N, K, y, y_dtype, stream);
  return launch_gemm(x, M, codes, scales, N, K, y, y_dtype == TB_BF16, false, 1, stream);
}

int gemm_splitk_parts(int64_t M, int64_t N, int64_t K) {
  // Each workgroup is latency bound: about one K step (64) per microsecond,
  // two per scale group.  Two workgroups fit a CU, so 512 run at once and a
  // launch takes ceil(workgroups / 512) rounds of ceil(G / S) groups each.
  // Each split beyond one adds M * N fp32 written and read back (about 5 TB/s)
  // and a second launch.  Take the S in 1 .. min(16, G) with the lowest
  // estimate (the smaller S on ties).
  const int64_t tiles = (N / BN) * ((M + BM - 1) / BM), G = K / kBlock;
  const int64_t smax = std::min<int64_t>(16, G);
  int best = 1;
  double best_us = 0.0;
  for (int64_t s = 1; s <= smax; ++s) {
    const int64_t rounds = (tiles * s + 511) / 512, groups = (G + s - 1) / s;
    double us = 2.2 * (double)(rounds * groups);
    if (s > 1) us += 2.0 + 8.0 * (double)s * (double)M * (double)N / 5.0e6;
    if (s == 1 || us < best_us) {
      best = (int)s;
      best_us = us;
    }
  }
  return best;
}

hipError_t launch_gemm_ternary_splitk(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                      int64_t N, int64_t K, void* y, int y_dtype, float* workspace,
                                      size_t workspace_bytes, bool rotate, hipStream_t stream) {
  if (!rotate && M <= kSkinnyMaxRows) return launch_gemm_skinny(x, M, codes, scales, N, K, y, y_dtype, stream);
  const size_t part = (size_t)M * (size_t)N * sizeof(float);
  const int S = (int)std::min<size_t>((size_t)gemm_splitk_parts(M, N, K), workspace ? workspace_bytes / part : 0);
  if (S <= 1) return launch_gemm(x, M, codes, scales, N, K, y, y_dtype == TB_BF16, rotate, 1, stream);
  const hipError_t e = launch_gemm(x, M, codes, scales, N, K, workspace, false, false, S, stream);
  if (e != hipSuccess) return e;
  const int64_t MN = M * N;
  if (rotate) {
    const int64_t blocks = std::min<int64_t>((MN / kBlock + 15) / 16, 4096);
    if (y_dtype == TB_BF16)
      hipLaunchKernelGGL((splitk_reduce_rot_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, workspace, S,
                         MN, y);
    else
      hipLaunchKernelGGL((splitk_reduce_rot_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, workspace, S,
                         MN, y);
    return hipGetLastError();
  }
  const int64_t blocks = std::min<int64_t>((MN / 4 + 255) / 256, 4096);
  if (y_dtype == TB_BF16)
    hipLaunchKernelGGL((splitk_reduce_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, workspace, S, MN, y);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, workspace, S, MN, y);
  return hipGetLastError();
}

}  // namespace tb
