// Ternary GEMM for at most 16 rows of activations (the mid-batch case between
// decode and prefill), the contraction of the prefill GEMM:
//   y[m][n] = sum_g f16(scale[n][g]) * sum_{k in g} t[n][k] * x[m][k]
//
// With M <= 16 the 128 x 128 tiles of the prefill kernel are mostly padding
// and too few to fill the GPU, and the run is bound by streaming the codes.
// Here one v_mfma_f32_16x16x32_bf16 row block holds all M rows (rows past M
// repeat row M - 1 and are never stored) and its 16 columns are the 16 weight
// rows of one code tile, so the decoded weights never leave registers:
//   * a lane (q = lane / 16, i = lane % 16) loads the two code words it owns
//     in the tile layout (row i, columns 32q .. 32q + 31 of the group) and
//     decodes them in place.  The sum over K does not care in which order the
//     K positions enter, so the m-th product of the group takes, in lane q,
//     columns 32q + 8m .. 32q + 8m + 7 of both operands.
//   * decode: masking a word with 0xCCCCCCCC leaves in every nibble the field
//     of one column as the 4-bit float 0, +2 or -2 (sign bit, lowest exponent
//     bit); the word shifted left by 2 and masked gives the other eight
//     columns.  v_cvt_scalef32_pk_bf16_fp4 turns one byte of it (two columns)
//     into a bf16 pair, exactly.
//   * the activations are read from global memory in full 128-byte lines
//     (16 lanes per row), written to a per-wave LDS tile with 16-byte chunk c
//     of row r at position c ^ r, and read back as matrix operands (16 lanes
//     read one chunk of 16 rows: 16 distinct positions, distinct banks).
//   * each group's products accumulate in fp32, then are added to the result
//     times the group's fp16 scale; the result is halved on the way out.
// Work split: a workgroup owns two code tiles (32 output columns) and the
// whole of K; its W waves take consecutive slices of the scale groups, each
// wave streams its slice for both tiles with the codes, scales and
// activations of the next step already in flight, and the W partial results
// are summed in LDS in wave order.  The slice boundaries depend only on K and
// on W, which depends only on N and K, so a row's result does not depend on M
// or on timing.  Waves of different workgroups start their slices at
// different groups, which spreads the activation reads over the L2 channels.
#include <algorithm>
#include <cstdint>

#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

constexpr int kTiles = 2;   // code tiles (16 weight rows each) per workgroup, one product per launch
// ... and in a grouped launch, where there are workgroups enough: each
// activation load then serves four tiles (a 27B layer's four products at
// M = 16: 55-57 us with two tiles, 43.5-45 us with four, 50-52 us with eight;
// a single 17408 x 5120 product: 13.3 us with two, 19.7 with four)
constexpr int kGroupedTiles = 4;
constexpr int kAhead = 2;   // steps (scale groups) in flight ahead of the one in use
// longest K: every buffer offset (at most 32 K bytes of activations, 16 K of
// code words) stays below 2^31
constexpr int64_t kSkinnyMaxK = (int64_t)1 << 26;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// the 16 fields of one dense code word as bf16 pairs (2t): out[0..3] hold
// columns 0-7 of the word, out[4..7] columns 8-15, in column order
__device__ __forceinline__ void decode_word(uint32_t w, uint32_t (&out)[8]) {
  const uint32_t a = w & 0xCCCCCCCCu, b = (w << 2) & 0xCCCCCCCCu;
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a, 1.0f, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a, 1.0f, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a, 1.0f, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a, 1.0f, 3));
  out[4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b, 1.0f, 0));
  out[5] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b, 1.0f, 1));
  out[6] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b, 1.0f, 2));
  out[7] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b, 1.0f, 3));
}

// Word 3 of a buffer resource: the 32-bit data format raw loads need (with
// the format left invalid every load returns zero).  A buffer load takes a
// wave-uniform resource and step offset in scalar registers and a 32-bit lane
// offset, so a step's addresses cost no vector arithmetic; an offset past the
// resource's size reads zero instead of memory.
constexpr int kBufferWord3 = 0x00020000;

// a resource over [base, base + bytes); base wave-uniform
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, kBufferWord3);
}

__device__ __forceinline__ bf16x8 pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

// LDS of one workgroup of W waves over TL tiles
template <int W, int TL>
struct SkinnyLds {
  f32x4 red[W][TL][64];                                    // each wave's partial result
  __attribute__((aligned(16))) uint32_t xlds[W][16 * 64];  // per wave: [row][chunk ^ row][4]
};

// Workgroup `wg` of one product: code tiles TL wg .. TL wg + TL - 1.
// M <= 16; K / 128 >= W; N a multiple of 16 TL.
template <int W, int TL>
__device__ __forceinline__ void skinny_product(const uint16_t* __restrict__ x, int M,
                                               const uint32_t* __restrict__ codes,
                                               const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                               void* __restrict__ y, bool out_bf16, int64_t wg,
                                               SkinnyLds<W, TL>& sm) {
  constexpr int kTiles = TL;
  auto& red = sm.red;
  auto& xlds = sm.xlds;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: slice bounds and bases in scalars
  const int li = lane & 15, q = lane >> 4;
  const int64_t G = K / kBlock;
  const int64_t t0 = wg * kTiles;
  // this wave's scale groups [gb, gb + ng)
  const int64_t gb = G * w / W;
  const int ng = (int)(G * (w + 1) / W - gb);
  // Loads through buffer resources based at group gb (the launchers keep
  // every offset below 2^31 bytes).  Activations: load m brings rows 4m + q
  // (clamped to M - 1), 16-byte chunk li of group gb + g, at byte
  // x_lane[m] + 256 g.  Code words of tile t0 + t, group gb + g: byte
  // 512 (t G + g) + 8 lane; scales [N/16][G][16], the lane's weight row li:
  // byte 32 (t G + g) + 2 li.
  const __amdgpu_buffer_rsrc_t xrs = buffer_over(x + gb * kBlock, ((int64_t)M * K - gb * kBlock) * 2);
  const __amdgpu_buffer_rsrc_t crs = buffer_over(codes + (t0 * G + gb) * 128, (kTiles * G - gb) * 512);
  const __amdgpu_buffer_rsrc_t srs = buffer_over(scales + (t0 * G + gb) * 16, (kTiles * G - gb) * 32);
  int x_lane[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) x_lane[m] = (int)((std::min(4 * m + q, M - 1) * K + 8 * li) * 2);
  uint32_t* xl = xlds[w];

  // a ring of kAhead register sets; step s (group (s + rot) % ng of the
  // slice) lives in set s % kAhead.  Loads for steps past the slice reload
  // its last group and are never used.
  u32x2 cw[kAhead][kTiles];
  uint16_t sw[kAhead][kTiles];
  u32x4 xv[kAhead][4];
  const int rot = (int)(wg % ng);
  auto load = [&](int s, int set) {
    int g = std::min(s, ng - 1) + rot;
    g = g >= ng ? g - ng : g;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      xv[set][m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, x_lane[m], 256 * g, 0));
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int tg = t * (int)G + g;
      cw[set][t] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(crs, 8 * lane, 512 * tg, 0));
      sw[set][t] = __builtin_amdgcn_raw_buffer_load_b16(srs, 2 * li, 32 * tg, 0);
    }
  };

  f32x4 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  auto step = [&](int set) {
    // the activations of the group through LDS: written as loaded, read as operands
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = 4 * m + q;
      *reinterpret_cast<u32x4*>(xl + row * 64 + 4 * (li ^ row)) = xv[set][m];
    }
    bf16x8 a[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      a[m] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + li * 64 + 4 * ((4 * q + m) ^ li)));
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      uint32_t b0[8], b1[8];
      decode_word(cw[set][t][0], b0);
      decode_word(cw[set][t][1], b1);
      f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], pack4(b0[0], b0[1], b0[2], b0[3]), zero, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], pack4(b0[4], b0[5], b0[6], b0[7]), p, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], pack4(b1[0], b1[1], b1[2], b1[3]), p, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], pack4(b1[4], b1[5], b1[6], b1[7]), p, 0, 0, 0);
      const float sc = (float)__builtin_bit_cast(_Float16, sw[set][t]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] = __builtin_fmaf(p[r], sc, acc[t][r]);
    }
  };

  // The scheduling barriers keep each set's loads in issue order between the
  // steps, so the wait before a step covers that set alone.  Whole trips of
  // kAhead steps, then the one step an odd slice has left (set 0), so that
  // every step taken is accumulated.
  static_assert(kAhead == 2, "the loop below leaves at most one step after its trips");
#pragma unroll
  for (int r = 0; r < kAhead; ++r) {
    load(r, r);
    __builtin_amdgcn_sched_barrier(0);
  }
  int s = 0;
  for (; s + kAhead <= ng; s += kAhead) {
#pragma unroll
    for (int r = 0; r < kAhead; ++r) {
      step(r);
      __builtin_amdgcn_sched_barrier(0);
      load(s + r + kAhead, r);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (s < ng) step(0);

  // lane holds acc[t][r] = 2 y[4q + r][16 (t0 + t) + li]
#pragma unroll
  for (int t = 0; t < kTiles; ++t) red[w][t][lane] = acc[t];
  __syncthreads();
  const float* rf = reinterpret_cast<const float*>(red);
  for (int e = threadIdx.x; e < kTiles * 256; e += 64 * W) {
    const int t = e >> 8, m = (e >> 4) & 15, n = e & 15;
    if (m >= M) continue;
    const int off = (t * 64 + (m >> 2) * 16 + n) * 4 + (m & 3);
    float v = rf[off];
#pragma unroll
    for (int ww = 1; ww < W; ++ww) v += rf[ww * kTiles * 256 + off];
    v *= 0.5f;
    const int64_t o = (int64_t)m * N + (t0 + t) * 16 + n;
    if (out_bf16)
      static_cast<uint16_t*>(y)[o] = (uint16_t)f32_to_bf16_rne(v);
    else
      static_cast<float*>(y)[o] = v;
  }
}

template <int W, bool OUT_BF16>
__global__ void __launch_bounds__(64 * W) gemm_skinny_kernel(const uint16_t* __restrict__ x, int M,
                                                            const uint32_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales, int64_t N,
                                                            int64_t K, void* __restrict__ y) {
  __shared__ SkinnyLds<W, kTiles> sm;
  skinny_product<W, kTiles>(x, M, codes, scales, N, K, y, OUT_BF16, blockIdx.x, sm);
}

// Several products in one launch: segment c owns workgroups [wg_begin,
// next segment's wg_begin).  The segment is found per workgroup from the
// kernel arguments (scalar compares).
struct SkinnySeg {
  const uint16_t* x;
  const uint32_t* codes;
  const uint16_t* scales;
  void* y;
  int64_t N, K;
  int M, out_bf16, wg_begin, reserved;
};

struct SkinnySegs {
  SkinnySeg s[TB_MAX_SEGMENTS];
  int count;
};

template <int W>
__global__ void __launch_bounds__(64 * W) gemm_skinny_multi_kernel(SkinnySegs segs) {
  __shared__ SkinnyLds<W, kGroupedTiles> sm;
  int seg = 0;
#pragma unroll
  for (int t = 1; t < TB_MAX_SEGMENTS; ++t)
    seg += (t < segs.count && (int)blockIdx.x >= segs.s[t].wg_begin) ? 1 : 0;
  const SkinnySeg& sg = segs.s[seg];
  skinny_product<W, kGroupedTiles>(sg.x, sg.M, sg.codes, sg.scales, sg.N, sg.K, sg.y, sg.out_bf16 != 0,
                                   (int)blockIdx.x - sg.wg_begin, sm);
}

template <int W>
hipError_t launch_w(const uint16_t* x, int M, const uint32_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                    void* y, bool bf16_out, hipStream_t stream) {
  const dim3 grid((unsigned)(N / 16 / kTiles)), block(64 * W);
  if (bf16_out)
    hipLaunchKernelGGL((gemm_skinny_kernel<W, true>), grid, block, 0, stream, x, M, codes, scales, N, K, y);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<W, false>), grid, block, 0, stream, x, M, codes, scales, N, K, y);
  return hipGetLastError();
}

}  // namespace

template <int W>
hipError_t launch_multi_w(const SkinnySegs& segs, unsigned wgs, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_skinny_multi_kernel<W>), dim3(wgs), dim3(64 * W), 0, stream, segs);
  return hipGetLastError();
}

int gemm_skinny_waves(int64_t N, int64_t K) {
  // Eight waves per workgroup while the workgroups fit on the compute units
  // at once (at most 256 of them), four beyond that (measured on the three
  // layer shapes at M = 16); never more waves than scale groups.
  const int64_t G = K / kBlock, wgs = N / 16 / kTiles;
  int w = wgs <= 256 ? 8 : 4;
  while (w > G) w /= 2;
  return w;
}

hipError_t launch_gemm_skinny(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                              int64_t N, int64_t K, void* y, int y_dtype, hipStream_t stream) {
  if (M < 1 || M > kSkinnyMaxRows || N % (16 * kTiles) != 0 || K % kBlock != 0 || K > kSkinnyMaxK)
    return hipErrorInvalidValue;
  const bool bf16 = y_dtype == TB_BF16;
  switch (gemm_skinny_waves(N, K)) {
    case 8: return launch_w<8>(x, (int)M, codes, scales, N, K, y, bf16, stream);
    case 4: return launch_w<4>(x, (int)M, codes, scales, N, K, y, bf16, stream);
    case 2: return launch_w<2>(x, (int)M, codes, scales, N, K, y, bf16, stream);
    default: return launch_w<1>(x, (int)M, codes, scales, N, K, y, bf16, stream);
  }
}

int gemm_skinny_multi_waves(const tb_gemm_segment* segs, int count) {
  // the single-product rule over the launch's workgroups; never more waves
  // than the shortest product's scale groups
  int64_t wgs = 0, gmin = INT64_MAX;
  for (int c = 0; c < count; ++c) {
    wgs += segs[c].N / 16 / kGroupedTiles;
    gmin = std::min<int64_t>(gmin, segs[c].K / kBlock);
  }
  int w = wgs <= 256 ? 8 : 4;
  while (w > gmin) w /= 2;
  return w;
}

hipError_t launch_gemm_skinny_multi(const tb_gemm_segment* segs, int count, hipStream_t stream) {
  if (count < 1 || count > TB_MAX_SEGMENTS) return hipErrorInvalidValue;
  // one product: the single launch (two tiles per workgroup is faster there)
  // and its result bit for bit
  if (count == 1)
    return launch_gemm_skinny(static_cast<const uint16_t*>(segs[0].x), segs[0].M, segs[0].codes, segs[0].scales,
                              segs[0].N, segs[0].K, segs[0].y, segs[0].y_dtype, stream);
  // The longest-K products take the first workgroups.  Their workgroups
  // carry the most work (a down projection's are 3.4 times a QKV's), and a
  // launch has more workgroups than fit on the GPU at once: dispatched first,
  // the long ones run beside the short ones, and the short ones left over go
  // to the compute units that free up first.  A 27B layer's four products at
  // M = 16: 43.4-44.5 -> 36.7-37.6 us.  A workgroup's result depends only on
  // its index within its own product, so the order changes no result.
  int ord[TB_MAX_SEGMENTS];
  for (int c = 0; c < count; ++c) ord[c] = c;
  std::stable_sort(ord, ord + count, [&](int a, int b) { return segs[a].K > segs[b].K; });
  SkinnySegs ss{};
  int64_t wgs = 0;
  for (int c = 0; c < count; ++c) {
    const tb_gemm_segment& a = segs[ord[c]];
    if (a.M < 1 || a.M > kSkinnyMaxRows || a.N % (16 * kGroupedTiles) != 0 || a.K % kBlock != 0 ||
        a.K > kSkinnyMaxK)
      return hipErrorInvalidValue;
    ss.s[c] = SkinnySeg{static_cast<const uint16_t*>(a.x), a.codes, a.scales, a.y, a.N, a.K, (int)a.M,
                        a.y_dtype == TB_BF16 ? 1 : 0, (int)wgs, 0};
    wgs += a.N / 16 / kGroupedTiles;
  }
  ss.count = count;
  if (wgs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  switch (gemm_skinny_multi_waves(segs, count)) {
    case 8: return launch_multi_w<8>(ss, (unsigned)wgs, stream);
    case 4: return launch_multi_w<4>(ss, (unsigned)wgs, stream);
    case 2: return launch_multi_w<2>(ss, (unsigned)wgs, stream);
    default: return launch_multi_w<1>(ss, (unsigned)wgs, stream);
  }
}

}  // namespace tb
