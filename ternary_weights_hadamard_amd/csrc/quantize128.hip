// Offline quantise/pack: per 128x128 block W' = H B H^T / 128, a scale and a
// threshold per 128-group (one row of a block), ternarise, pack.  Rules: the
// absmean scale with threshold s/2 (dense, 2:4), or the error-minimising
// threshold and scale (dense): over the group's magnitudes theta, the kept set
// {|w'| >= theta} with the largest S^2 / j (S its magnitude sum, j its size),
// scale S / j, which minimises ||w' - s t||^2; ties to the larger theta.
//
// Method: mhpq.cn/news/1159370 §1.1 (scale = the group's mean absolute value;
// divide, round, clip to {-1, 0, 1}), §1.2 (2:4: keep two of four, ternarise
// the survivors), §1.3 (one fp16 scale per 128 elements), §3.1 (2 bits per
// weight); dpshk.com/news/5289456 §2.1 and §3.2 (transform per 128x128 block,
// then sign(w) * (|w| > thr)).
//
// One workgroup of 256 threads owns one block:
//   phase A  thread (column c, row half h) loads 64 rows of one column with
//            coalesced 128-byte row segments and runs the column transform:
//            6 butterfly rounds in registers, the 7th across lane ^ 32 with
//            v_permlane32_swap; the block goes to LDS (fp32, 67.6 KB);
//   phase B  thread (row r, column half h) reads 64 contiguous columns of its
//            row with 16-byte LDS reads and runs the row transform the same
//            way.  Each thread now holds 64 consecutive K-elements of one row:
//            the group's |.| sum is an in-register sum plus one exchange, and
//            the codes of 64 elements pack into four whole words (two word
//            pairs of the row's 16 x 128 tile).
// The 1/128 of the 2D transform is a power of two; it is folded into the
// threshold and the stored scale instead of being applied to every element.
// The two-plane format ternarises the group once, subtracts the stored scale
// times the codes (the residual calibration of xxqk.cn/news/652513 §3) and
// ternarises that residual by the same rule into the next group slot.
// The error-minimising rule evaluates every magnitude of the group as a
// threshold: lane pair (l, l ^ 32) holds the group, exchanges one candidate of
// each lane per step and adds both lanes' kept counts and sums.
#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

constexpr int kLdsStride = kBlock + 4;  // floats per LDS row (bank spread for 16-byte reads)

// In-register butterflies over the six low index bits of 64 values.
__device__ __forceinline__ void fwht64_regs(float (&v)[64]) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      if ((e & h) == 0) {
        float a = v[e], c = v[e + h];
        v[e] = a + c;
        v[e + h] = a - c;
      }
    }
  }
}

// Butterfly round over lane bit 5 (the 7th index bit): lanes 0-31 hold index
// bit 6 = 0 and get own + partner, lanes 32-63 get partner - own.
__device__ __forceinline__ void fwht_cross_halves(float (&v)[64], float sgn) {
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    float lo, hi;
    swap_halves(v[e], lo, hi);
    v[e] = lo + sgn * hi;
  }
}

// 2-bit field position of column offset r (0..15) inside a dense code word:
// r < 8 in bits 2-3 of nibble r, r >= 8 in bits 0-1 of nibble r - 8.
__device__ __forceinline__ constexpr int field_pos(int r) { return 4 * (r & 7) + 2 - 2 * (r >> 3); }

enum Rule { kAbsmean = 0, kTwoFour = 1, kMinError = 2, kResidual = 3 };

template <int RULE>
__global__ void __launch_bounds__(256, 2) quantize128_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                           uint32_t* __restrict__ codes,
                                                           uint32_t* __restrict__ meta,
                                                           uint16_t* __restrict__ scales,
                                                           int32_t* __restrict__ err_flag) {
  __shared__ float lds[kBlock * kLdsStride];
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;      // lane bit 5
  const int col = 32 * wv + (lane & 31);
  const float sgn = half ? -1.f : 1.f;
  const int64_t kblocks = K / kBlock;
  const int64_t nblk = (N / kBlock) * kblocks;

  // one block per workgroup (a loop over blocks made the compiler keep the
  // 64 load addresses across it, spilled to scratch)
  {
    const int64_t blk = blockIdx.x;
    if (blk >= nblk) return;
    const int64_t n0 = (blk / kblocks) * kBlock;
    const int64_t bk = blk % kblocks;
    const int64_t k0 = bk * kBlock;
    uint32_t flags = 0;

    // ---- phase A: column transform (along N) ----
    // addresses: the block's row i (wave-uniform) plus a 32-bit lane offset
    float v[64];
    {
      const float* base = W + n0 * K + k0;
      const int lane_off = 64 * half * (int)K + col;  // < 64 K + 128 floats
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = __builtin_nontemporal_load(base + (int64_t)i * K + lane_off);
    }
    fwht64_regs(v);
    fwht_cross_halves(v, sgn);
    {
      // row r = 64*half + i; XOR-swizzle the column by row bit 6 to spread banks
      const int pc = col ^ (half << 5);
#pragma unroll
      for (int i = 0; i < 64; ++i) lds[(64 * half + i) * kLdsStride + pc] = v[i];
    }
    __syncthreads();

    // ---- phase B: row transform (along K) ----
    const int row = 32 * wv + (lane & 31);
    {
      const int sw = ((row >> 6) & 1) << 5;
      const float* rp = lds + row * kLdsStride;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(rp + ((64 * half + 4 * q) ^ sw));
        v[4 * q] = t4[0];
        v[4 * q + 1] = t4[1];
        v[4 * q + 2] = t4[2];
        v[4 * q + 3] = t4[3];
      }
    }
    fwht64_regs(v);
    fwht_cross_halves(v, sgn);
    // v[j] = T[row][64*half + j] with T = H B H^T (unnormalised: W' = T / 128).
    // Every element of T is a +- sum over a whole row and column of the block,
    // so one non-finite weight makes every element non-finite: one test per
    // thread on a sum of its values replaces a test per loaded weight (three
    // instructions per weight, a tenth of the kernel's).  A finite block
    // whose transform overflows fp32 is flagged the same way.

    const int64_t grow = n0 + row;
    if constexpr (RULE == kMinError || RULE == kTwoFour) {
      float chk = 0.f;
#pragma unroll
      for (int j = 0; j < 64; ++j) chk += __builtin_fabsf(v[j]);
      if (!__builtin_isfinite(chk)) flags |= TB_EFLAG_NONFINITE;
    }
    if constexpr (RULE == kMinError) {
      // every magnitude of the group is a candidate threshold; per step each
      // lane of the pair offers one, both lanes count and sum their own
      // magnitudes >= each candidate, and the pair adds its halves
      float best_e = -1.f, best_th = 0.f, best_s = 0.f, best_j = 1.f;
#pragma unroll 1
      for (int i = 0; i < 64; ++i) {
        // candidate i of this lane, picked with selects (an indexed read would
        // move v to scratch memory)
        float cand = 0.f;
#pragma unroll
        for (int e = 0; e < 64; ++e) cand = e == i ? v[e] : cand;
        float th_lo, th_hi;
        swap_halves(__builtin_fabsf(cand), th_lo, th_hi);
        float c_lo = 0.f, s_lo = 0.f, c_hi = 0.f, s_hi = 0.f;
#pragma unroll
        for (int e = 0; e < 64; ++e) {
          const float x = __builtin_fabsf(v[e]);
          const bool g_lo = x >= th_lo, g_hi = x >= th_hi;
          c_lo += g_lo ? 1.f : 0.f;
          s_lo += g_lo ? x : 0.f;
          c_hi += g_hi ? 1.f : 0.f;
          s_hi += g_hi ? x : 0.f;
        }
        // totals over the pair (the same two terms in both lanes, so the same sums)
        float a0, a1, b0, b1, d0, d1, f0, f1;
        swap_halves(c_lo, a0, a1);
        swap_halves(s_lo, b0, b1);
        swap_halves(c_hi, d0, d1);
        swap_halves(s_hi, f0, f1);
        const float cl = a0 + a1, sl = b0 + b1, ch = d0 + d1, sh = f0 + f1;
        const float el = sl * sl / cl, eh = sh * sh / ch;
        if (el > best_e || (el == best_e && th_lo > best_th)) { best_e = el; best_th = th_lo; best_s = sl; best_j = cl; }
        if (eh > best_e || (eh == best_e && th_hi > best_th)) { best_e = eh; best_th = th_hi; best_s = sh; best_j = ch; }
      }
      const float s = best_s / best_j * 0.0078125f;  // mean kept |T| / 128
      u32x4 words = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        const uint32_t nz = (__builtin_fabsf(v[j]) >= best_th && v[j] != 0.f) ? 1u : 0u;
        const uint32_t ng = (nz && v[j] < 0.f) ? 2u : 0u;
        words[j >> 4] |= (nz | ng) << field_pos(j & 15);
      }
      uint32_t* tile = codes + ((grow >> 4) * kblocks + bk) * 128 + 2 * (grow & 15);
      *reinterpret_cast<u32x2*>(tile + 64 * half) = u32x2{words[0], words[1]};
      *reinterpret_cast<u32x2*>(tile + 64 * half + 32) = u32x2{words[2], words[3]};
      if (half == 0) {
        const uint32_t h16 = f32_to_f16_bits(s);
        if ((h16 & 0x7fffu) == 0x7c00u) flags |= TB_EFLAG_SCALE_OVF;
        scales[((grow >> 4) * kblocks + bk) * 16 + (grow & 15)] = (uint16_t)h16;
      }
    } else if constexpr (RULE == kAbsmean || RULE == kResidual) {
      // one plane, or two with their groups interleaved (group 2 bk + p)
      constexpr int kPlanes = RULE == kResidual ? 2 : 1;
#pragma unroll
      for (int p = 0; p < kPlanes; ++p) {
        float asum = 0.f;
#pragma unroll
        for (int j = 0; j < 64; ++j) asum += __builtin_fabsf(v[j]);
        if (p == 0 && !__builtin_isfinite(asum)) flags |= TB_EFLAG_NONFINITE;
        float lo, hi;
        swap_halves(asum, lo, hi);
        const float tsum = lo + hi;               // sum over the 128-group of |T|
        const float thr = tsum * 0.00390625f;     // |W'| > s/2  <=>  |T| > sum|T| / 256
        const float s = tsum * 6.103515625e-05f;  // s = sum|T| / 128 / 128
        u32x4 words = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          const uint32_t nz = __builtin_fabsf(v[j]) > thr ? 1u : 0u;
          const uint32_t ng = (nz && v[j] < 0.f) ? 2u : 0u;
          words[j >> 4] |= (nz | ng) << field_pos(j & 15);
        }
        // columns 64 half + j of group bk: word pairs of lane groups 2 half and 2 half + 1
        const int64_t gcol = kPlanes * bk + p;
        uint32_t* tile = codes + ((grow >> 4) * kPlanes * kblocks + gcol) * 128 + 2 * (grow & 15);
        *reinterpret_cast<u32x2*>(tile + 64 * half) = u32x2{words[0], words[1]};
        *reinterpret_cast<u32x2*>(tile + 64 * half + 32) = u32x2{words[2], words[3]};
        const uint32_t h16 = f32_to_f16_bits(s);
        if (half == 0) {
          if ((h16 & 0x7fffu) == 0x7c00u) flags |= TB_EFLAG_SCALE_OVF;
          scales[((grow >> 4) * kPlanes * kblocks + gcol) * 16 + (grow & 15)] = (uint16_t)h16;
        }
        if (p + 1 < kPlanes) {
          // the residual against the stored scale, in units of T: T - 128 f16(s) t
          const float s128 = f16_bits_to_f32(h16) * 128.f;
#pragma unroll
          for (int j = 0; j < 64; ++j) {
            const float a = __builtin_fabsf(v[j]) > thr ? s128 : 0.f;
            v[j] = v[j] < 0.f ? v[j] + a : v[j] - a;
          }
        }
      }
    } else {
      // 2:4: in each quad keep the two largest |T|, ties to the lower position
      float ksum = 0.f;
      uint32_t nib[16];
      uint32_t sbits = 0;
#pragma unroll
      for (int qd = 0; qd < 16; ++qd) {
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = __builtin_fabsf(v[4 * qd + e]);
        bool keep[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int beaten = 0;
#pragma unroll
          for (int f = 0; f < 4; ++f)
            if (f != e) beaten += (a[f] > a[e] || (a[f] == a[e] && f < e)) ? 1 : 0;
          keep[e] = beaten < 2;
        }
        // exactly two are kept: the first is at 0..2, the second at 1..3
        const uint32_t i0 = keep[0] ? 0u : (keep[1] ? 1u : 2u);
        const uint32_t i1 = keep[3] ? 3u : (keep[2] ? 2u : 1u);
        const float v0 = keep[0] ? v[4 * qd] : (keep[1] ? v[4 * qd + 1] : v[4 * qd + 2]);
        const float v1 = keep[3] ? v[4 * qd + 3] : (keep[2] ? v[4 * qd + 2] : v[4 * qd + 1]);
        ksum += __builtin_fabsf(v0) + __builtin_fabsf(v1);
        nib[qd] = i0 | (i1 << 2);
        sbits |= (v0 < 0.f ? 1u : 0u) << qd;
        sbits |= (v1 < 0.f ? 1u : 0u) << (16 + qd);
      }
      float lo, hi;
      swap_halves(ksum, lo, hi);
      const float s = (lo + hi) * 0.0001220703125f;  // mean over 64 kept of |T|/128
      u32x2 mw = {0u, 0u};
#pragma unroll
      for (int qd = 0; qd < 16; ++qd) mw[qd >> 3] |= nib[qd] << (4 * (qd & 7));
      // lane-major blocks of four groups: this thread holds lanes 16 q + i for
      // q = 2 half, 2 half + 1 (row i of the tile) of group bk = 4 b + j: meta
      // word j of each lane, its 16-bit sign field (the byte pair of sbits at
      // bits 8 (q % 2) and 16 + 8 (q % 2)) in half j % 2 of sign word j / 2,
      // and the row's scale at [b][i / 4][j][i % 4].  The last group of K also
      // zeroes the padded groups of its block.
      const int64_t g4 = (kblocks + 3) >> 2;
      const int64_t tb = (grow >> 4) * g4 + (bk >> 2);
      const int ri = (int)(grow & 15), j = (int)(bk & 3);
      uint16_t* sfield = reinterpret_cast<uint16_t*>(codes);
      const uint32_t f0 = (sbits & 0xFFu) | (((sbits >> 16) & 0xFFu) << 8);
      const uint32_t f1 = ((sbits >> 8) & 0xFFu) | (((sbits >> 24) & 0xFFu) << 8);
      const int64_t l0 = tb * 64 + 16 * (2 * half) + ri, l1 = l0 + 16;
      meta[l0 * 4 + j] = mw[0];
      meta[l1 * 4 + j] = mw[1];
      sfield[l0 * 4 + j] = (uint16_t)f0;
      sfield[l1 * 4 + j] = (uint16_t)f1;
      const uint32_t h16 = f32_to_f16_bits(s);
      if (half == 0) {
        if ((h16 & 0x7fffu) == 0x7c00u) flags |= TB_EFLAG_SCALE_OVF;
        scales[tb * 64 + ((ri >> 2) * 4 + j) * 4 + (ri & 3)] = (uint16_t)h16;
      }
      if (bk == kblocks - 1) {
        for (int jj = j + 1; jj < 4; ++jj) {
          meta[l0 * 4 + jj] = 0u;
          meta[l1 * 4 + jj] = 0u;
          sfield[l0 * 4 + jj] = 0;
          sfield[l1 * 4 + jj] = 0;
          if (half == 0) scales[tb * 64 + ((ri >> 2) * 4 + jj) * 4 + (ri & 3)] = 0;
        }
      }
    }
    wave_flag_or(err_flag, flags);
  }
}

}  // namespace

hipError_t launch_quantize128(const float* W, int64_t N, int64_t K, int fmt, uint32_t* codes, uint32_t* meta,
                              uint16_t* scales, int32_t* err_flag, hipStream_t stream) {
  const int64_t nblk = (N / kBlock) * (K / kBlock);
  // one workgroup per 128 x 128 block
  if (nblk * 256 >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)nblk;
  if (fmt == TB_FMT_24)
    hipLaunchKernelGGL((quantize128_kernel<kTwoFour>), dim3(grid), dim3(256), 0, stream, W, N, K, codes, meta,
                       scales, err_flag);
  else if (fmt == TB_FMT_DENSE_MINERR)
    hipLaunchKernelGGL((quantize128_kernel<kMinError>), dim3(grid), dim3(256), 0, stream, W, N, K, codes, meta,
                       scales, err_flag);
  else if (fmt == TB_FMT_DENSE_RESID)
    hipLaunchKernelGGL((quantize128_kernel<kResidual>), dim3(grid), dim3(256), 0, stream, W, N, K, codes, meta,
                       scales, err_flag);
  else
    hipLaunchKernelGGL((quantize128_kernel<kAbsmean>), dim3(grid), dim3(256), 0, stream, W, N, K, codes, meta,
                       scales, err_flag);
  return hipGetLastError();
}

}  // namespace tb
