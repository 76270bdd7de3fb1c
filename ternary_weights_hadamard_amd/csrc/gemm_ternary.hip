// Prefill GEMM with dense ternary weights, the decode contraction for M rows:
//   y[m][n] = sum_g f16(scale[n][g]) * sum_{k in g} t[n][k] * x[m][k]
//
// The one dense contraction of the path, so it runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16) with bf16 operands: the activations as they are,
// each weight as the bf16 value 2t (exact; the result is halved on the way
// out).
// Tiling: 64 x 256 output tile per workgroup of 4 waves; wave w owns columns
// 64 w .. 64 w + 63 (four 16-column code tiles) for all 64 rows.  Only the
// activations are staged in LDS (double-buffered K steps of 64); each wave
// loads its own code words and decodes them straight into matrix operands
// with v_cvt_scalef32_pk_bf16_fp4 (a code field masked into bits 2-3 of a
// nibble is the e2m1 value of 2t), so no weight passes through LDS.  An LDS
// row is 128 bytes, eight 16-byte chunks; chunk c of row r is stored at
// c ^ F(r), F(r) = (r ^ (((r >> 2) ^ (r >> 3)) & 1)) & 7: the operand reads
// (16 lanes read one chunk of 16 consecutive rows) touch distinct banks
// whether the LDS serves 8 lanes from 32 banks or 16 lanes from 64, and the
// tile writes at most two lanes per bank (checked by enumeration).
// Scales: the accumulators hold the sum so far in units of the column's last
// nonzero group scale; a group with scale s first rescales them by
// unit / s, then adds its products, and a zero-scale group's code fields are
// masked to zero.  With one set of accumulators a wave needs about 156
// registers, so three workgroups share a CU.  The rescale factor is rounded
// (exact for power-of-two scales), about 2^-23 relative per group.
// Rotated output (ROT): the back-rotation y = R_N y' (the second transform of
// dpshk.com/news/5289456 §4.2, fused with the product) runs in the epilogue:
// the tile goes to LDS in fp32, each 16-lane group transforms one 128-column
// block of a row with the in-register butterflies of the activation
// transform, and the result is rounded once.
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

constexpr int KT = 64;       // K per step
constexpr int kMaxSplits = 16;  // split-K parts, at most
constexpr int LDS_ROW = KT;  // bf16 elements per LDS row (128 bytes, chunks swizzled)

// element offset of (row r, element k) in a swizzled LDS tile
__device__ __forceinline__ int lds_off(int r, int k) {
  const int f = (r ^ (((r >> 2) ^ (r >> 3)) & 1)) & 7;
  return r * LDS_ROW + ((((k >> 3) ^ f) & 7) << 3) + (k & 7);
}

// K order: in a 64-K step, lane (i, q) takes one whole code word per tile -
// K 16 q .. 16 q + 15 of the step, the word of half q / 2 and slot q % 2 - and
// feeds its first eight K to the step's first instruction and the other eight
// to the second; the activation operand reads the same K (LDS chunk 2 q + kk
// of its row).  The two instructions of a step thus split its 64 K
// differently from a plain order; a group's four cover the same 128 K.
// Against the previous design (128 x 128 tiles, weights decoded once per
// workgroup into LDS and read back by every wave, LDS bound), M = 2048 on the
// 27B FFN shapes: 905 -> 1210 TFLOP/s at K = 5120, 876 -> 1179 at K = 17408.
constexpr int RBM = 64, RBN = 256;
constexpr int kRCodeRing = 4;  // steps of code words in flight (two groups)
constexpr int RTROW = 128 + 4;  // fp32 elements per row of the rotation epilogue's tile (one 128-block)

template <bool OUT_BF16, bool ROT>
__global__ void __launch_bounds__(256, 3) gemm_rw_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                      const uint32_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                                      void* __restrict__ y, int splits) {
  constexpr int kXStage = RBM * LDS_ROW;  // bf16 elements of one activation stage
  constexpr int kLdsElems = ROT && RBM * RTROW * 2 > 2 * kXStage ? RBM * RTROW * 2 : 2 * kXStage;
  static_assert(RBN == 256, "the rotation epilogue takes the tile's two 128-column blocks in turn");
  __shared__ __attribute__((aligned(16))) uint16_t lds_mem[kLdsElems];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, q = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * RBM;
  const int64_t n0 = (int64_t)blockIdx.x * RBN;
  const int64_t G = K / kBlock;
  const int64_t gb = G * blockIdx.z / splits, ge = G * (blockIdx.z + 1) / splits;
  const int ngroups = (int)(ge - gb), nsteps = 2 * ngroups;

  // this wave's four code tiles.  N is a multiple of 128, so in the last
  // workgroup a wave's tiles are all inside N or all past it; a wave past N
  // reads the last four tiles instead (its results are never stored).
  const int64_t ntiles = N >> 4;
  const int64_t ct0 = std::min<int64_t>((n0 >> 4) + 4 * wv, ntiles - 4);
  // Addresses are a wave-uniform pointer (scalar registers) plus a 32-bit
  // lane offset fixed for the whole loop, so a load needs no 64-bit vector
  // address arithmetic.  Code word of (tile ct0 + j, group gb + g, step h of
  // the group) for this lane: cbase + j ctile + 128 g + 64 h + coff.
  const uint32_t* cbase = codes + (ct0 * G + gb) * 128;
  const int coff = 32 * (q >> 1) + 2 * li + (q & 1);
  const int64_t ctile = G * 128;  // words between consecutive tiles
  const _Float16* sbase = reinterpret_cast<const _Float16*>(scales) + (ct0 * G + gb) * 16;

  // activation staging: thread -> row tid / 4, 16 consecutive K at 16 (tid % 4);
  // rows past M read row M - 1 (they reach only output rows never stored)
  const int xr = tid >> 2, xk = (tid & 3) * 16;
  const uint16_t* xbase = x + m0 * K + gb * kBlock;  // wave-uniform
  const int xoff = (int)std::min<int64_t>(xr, M - 1 - m0) * (int)K + xk;  // < 64 K elements

  // Register rings, indexed by compile-time slots (the caller passes the
  // step's place in a four-step trip): with an index the compiler cannot
  // resolve, it copies loaded values between registers and waits for loads
  // just issued.
  u32x4 xs[2][2];             // [step parity] 16 bf16 of row xr
  uint32_t cw[kRCodeRing][4];  // [step % kRCodeRing] one code word per tile
  _Float16 sw[2][4];          // [group parity] scale per tile
  auto gload_x = [&](int step, int par) {
    const uint16_t* src = xbase + (int64_t)std::min(step, nsteps - 1) * KT;
    xs[par][0] = *reinterpret_cast<const u32x4*>(src + xoff);
    xs[par][1] = *reinterpret_cast<const u32x4*>(src + xoff + 8);
  };
  auto gload_w = [&](int step, int slot) {  // steps past the range reload the last (never used)
    const int st = std::min(step, nsteps - 1);
    const uint32_t* src = cbase + (int64_t)(st >> 1) * 128 + 64 * (st & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) cw[slot][j] = (src + j * ctile)[coff];
  };
  auto gload_s = [&](int g, int par) {
    const _Float16* src = sbase + (int64_t)std::min(g, ngroups - 1) * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) sw[par][j] = (src + j * G * 16)[li];
  };
  auto lstore = [&](int par) {
    uint16_t* d = lds_mem + par * kXStage;
    *reinterpret_cast<u32x4*>(d + lds_off(xr, xk)) = xs[par][0];
    *reinterpret_cast<u32x4*>(d + lds_off(xr, xk + 8)) = xs[par][1];
  };

  // acc holds the sum so far in units of `unit` (per column: the last
  // nonzero group scale); a group with scale s rescales it by unit / s
  // before its products are added, and a zero-scale group adds nothing (its
  // code fields are masked to zero)
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float unit[4] = {1.f, 1.f, 1.f, 1.f};
  uint32_t fmask[4];  // 0xCCCCCCCC, or 0 for a zero-scale group

  // the products of one step (c: its place in the trip) from activation stage
  // c & 1 and the code words of ring slot c
  float rs[4];  // per tile: the rescale factor of the group that starts at this step
  auto mfma_step = [&](int c) {
    const uint16_t* xa = lds_mem + (c & 1) * kXStage;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(xa + lds_off(16 * i + li, 16 * q + 8 * kk));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = cw[c][j];
        const uint32_t f = (kk == 0 ? w : w << 2) & fmask[j];  // e2m1 fields of 2t
        b[j] = __builtin_bit_cast(
            bf16x8, u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, 1.0f, 0)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, 1.0f, 1)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, 1.0f, 2)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, 1.0f, 3))});
      }
      // at a group's first step each accumulator is rescaled just before its
      // first product, so the multiplies interleave with the products of the
      // others instead of holding the matrix cores (27B FFN shapes at M =
      // 2048: about 1 % faster than rescaling all sixteen first)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if ((c & 1) == 0 && kk == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] *= rs[j];
          }
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
  };

  // one K step (step = 4 trip + c): at the start of a group the rescale
  // factors; its products; the code words of step + kRCodeRing into the freed ring slot;
  // at the end of a group the scales two groups on; the next step's
  // activations into the other stage and the step after that into the freed
  // registers; one barrier.  Steps past the range (an odd last trip) load
  // as the others but add nothing.
  auto step_body = [&](int step, int c) {
    const int par = c >> 1;  // group parity
    if (step < nsteps) {
      if ((c & 1) == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sg = (float)sw[par][j];
          const bool nz = sg != 0.f;
          rs[j] = nz ? unit[j] * __builtin_amdgcn_rcpf(sg) : 1.f;
          unit[j] = nz ? sg : unit[j];
          fmask[j] = nz ? 0xCCCCCCCCu : 0u;
        }
      }
      mfma_step(c);
    }
    gload_w(step + kRCodeRing, c);
    if (c & 1) gload_s((step >> 1) + 2, par);
    if (step + 1 < nsteps) lstore((c + 1) & 1);
    gload_x(step + 3, (c + 1) & 1);
    __syncthreads();
  };

#pragma unroll
  for (int c = 0; c < kRCodeRing; ++c) gload_w(c, c);
  gload_s(0, 0);
  gload_s(1, 1);
  gload_x(0, 0);
  lstore(0);
  gload_x(1, 1);
  gload_x(2, 0);
  __syncthreads();
  // two groups (four steps) per trip, every load unconditional: a branch
  // around the second group made the compiler merge the rings' registers
  // with copies that waited for loads it had just issued
  for (int t = 0; 2 * t < ngroups; ++t) {
    step_body(4 * t, 0);
    step_body(4 * t + 1, 1);
    step_body(4 * t + 2, 2);
    step_body(4 * t + 3, 3);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] *= unit[j];

  // lane holds acc[i][j][r] = 2 * y[m0 + 16i + 4q + r][n0 + 64 wv + 16j + li]
  const bool wave_live = (n0 >> 4) + 4 * wv < ntiles;
  if constexpr (ROT) {
    // The tile's two 128-column blocks in turn (waves 2 blk and 2 blk + 1 own
    // block blk), each through LDS in fp32 with padded rows; each 16-lane
    // group rotates one row of the block.  One block at a time keeps the
    // epilogue's LDS at 33.8 KB, so three workgroups share a CU (the whole
    // tile at once, 66.5 KB, allowed two).  The main loop's last barrier has
    // passed.
    float* t = reinterpret_cast<float*>(lds_mem);
    const int sub = tid & 15;
    for (int blk = 0; blk < 2; ++blk) {
      if ((wv >> 1) == blk) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              t[(16 * i + 4 * q + r) * RTROW + 64 * (wv & 1) + 16 * j + li] = acc[i][j][r] * 0.5f;
      }
      __syncthreads();
      // 64 rows, 16 per round of the workgroup's 16 groups: every wave runs 4 rounds
      for (int row = tid >> 4; row < RBM; row += 16) {
        const float* src = t + row * RTROW + 8 * sub;
        const f32x4 a = *reinterpret_cast<const f32x4*>(src);
        const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
        float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        fwht128_lanes(v, sub);
        const int64_t m = m0 + row;
        if (m >= M || n0 + 128 * blk >= N) continue;
        const int64_t base = m * N + n0 + 128 * blk + 8 * sub;
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
      __syncthreads();  // the block's reads are done before the next block's writes
    }
    return;
  }
  if (!wave_live) return;
  if (splits > 1) y = static_cast<float*>(y) + (size_t)blockIdx.z * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + 16 * i + 4 * q + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + 64 * wv + 16 * j + li;
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
    // every partial's load is issued before the first add (S <= kMaxSplits)
    f32x4 p[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
      if (s < S) p[s] = *reinterpret_cast<const f32x4*>(part + (size_t)s * MN + e);
    f32x4 a = p[0];
#pragma unroll
    for (int s = 1; s < kMaxSplits; ++s)
      if (s < S) {
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] += p[s][r];
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
      // every partial's loads are issued before the first add (S <= kMaxSplits)
      f32x4 pa[kMaxSplits], pb[kMaxSplits];
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s)
        if (s < S) {
          pa[s] = *reinterpret_cast<const f32x4*>(part + (size_t)s * MN + e);
          pb[s] = *reinterpret_cast<const f32x4*>(part + (size_t)s * MN + e + 4);
        }
      a = pa[0];
      b = pb[0];
#pragma unroll
      for (int s = 1; s < kMaxSplits; ++s)
        if (s < S) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            a[r] += pa[s][r];
            b[r] += pb[s][r];
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
  const int64_t mt = (M + RBM - 1) / RBM;
  if (mt > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + RBN - 1) / RBN), (unsigned)mt, (unsigned)splits), block(256);
#define TB_GEMM(B_, R_) \
  hipLaunchKernelGGL((gemm_rw_kernel<B_, R_>), grid, block, 0, stream, x, M, codes, scales, N, K, y, splits)
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
  // Time model of S splits (us), fitted to the 64 x 256 kernel on the
  // 27B-shaped layers (M = 17 .. 2048): a workgroup costs about 8 us of
  // launch, prologue and epilogue, then its ceil(G / S) scale groups take at
  // least 1.25 us each (one workgroup alone on a CU), or 0.83 us each per
  // workgroup sharing a CU; S > 1 adds the reduction launch, which reads the
  // S fp32 partials (about 6 TB/s) and pays about 0.5 us per partial.  Take
  // the S in 1 .. min(16, G) with the lowest estimate (the smaller on ties).
  const int64_t tiles = ((N + RBN - 1) / RBN) * ((M + RBM - 1) / RBM), G = K / kBlock;
  const int64_t smax = std::min<int64_t>(16, G);
  int best = 1;
  double best_us = 0.0;
  for (int64_t s = 1; s <= smax; ++s) {
    const double groups = (double)((G + s - 1) / s), per_cu = (double)((tiles * s + 255) / 256);
    double us = 8.0 + std::max(1.25 * groups, 0.83 * per_cu * groups);
    if (s > 1) us += 2.0 + 4.0 * (double)s * (double)M * (double)N / 6.0e6 + 0.5 * (double)s;
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
