// Blockwise 128-point orthonormal Walsh-Hadamard transform along K.
//
// xxqk.cn/news/652513 §2 computes the transform as log2(n) rounds of
// (a + b, a - b) butterflies; dpshk.com/news/5289456 §2.3 normalises by
// 1/sqrt(block size).  One 128-block lives in 16 consecutive lanes of a wave,
// 8 contiguous elements per lane (one 16-byte bf16 load), and the butterflies
// run in registers (fwht_lanes.h).  The kernel is HBM bound: 4 bytes per
// element for bf16 in and out.  Workgroups are one wave (four blocks): at
// decode sizes (a few hundred blocks) a launch is latency bound, and spreading
// it over more CUs took 0.2 us off each launch (3.9 -> 3.7 us for a 27B
// layer's four input rotations); prefill sizes are unchanged.
//
// With the act8 output the rounded bf16 result is re-encoded in the same pass
// as the dense GEMV's activation operand (act8.h); the same kernel without the
// transform re-encodes bf16 activations as they are.
#include "act8.h"
#include "fwht_lanes.h"
#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

enum OutKind { kOutF32 = 0, kOutBF16 = 1, kOutAct8 = 2 };

// A launch covers up to TB_MAX_SEGMENTS independent arrays (segments); the
// 128-blocks are numbered across them, each segment starting at a multiple
// of 4, so that the four blocks of a wave always lie in one segment.  The
// segment is then found per wave (scalar compares and loads of the kernel
// arguments); a per-lane choice kept all segments' pointers live and spilled
// them through VGPR lanes.  Segments may differ in their input and output
// dtypes (`kind`): a layer's outputs in fp32 rotated back and the next
// layer's bf16 inputs rotated and encoded, in one launch.
struct FwhtSeg {
  const void* x;
  void* y;
  int64_t nblocks, begin;
  int kind;   // 3 * (x bf16 ? 1 : 0) + OutKind
  int parts;  // fp32 input only: x holds `parts` partial arrays, added in order first
};

struct FwhtSegs {
  FwhtSeg s[TB_MAX_SEGMENTS];
  int count;
  int64_t total;
};

// One 128-block per 16 lanes: block b of a segment of nblocks blocks; lanes
// past the end (b >= nblocks) run the cross-lane rounds on zeros and store
// nothing.  An fp32 input of `parts` > 1 partial arrays (nblocks blocks
// apart) is their sum, taken in part order.
template <bool IN_BF16, int OUT, bool XFORM>
__device__ __forceinline__ void fwht_block(const void* x, void* y, int64_t nblocks, int64_t b, int sub,
                                           int parts = 1) {
  const bool live = b < nblocks;
  const int64_t base = b * kBlock + sub * 8;
  float v[8];
  if constexpr (IN_BF16) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (live) w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + base);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  } else {
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      // every part's loads are issued before the first add (a loop that adds
      // as it loads waits for one memory round trip per part: a 27B layer's
      // boundary rotation with four parts per output took 4.8 us)
      f32x4 pa[TB_MAX_PARTS], pc[TB_MAX_PARTS];
#pragma unroll
      for (int pp = 0; pp < TB_MAX_PARTS; ++pp) {
        if (pp < parts) {
          const f32x4* pn =
              reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + pp * nblocks * kBlock + base);
          pa[pp] = pn[0];
          pc[pp] = pn[1];
        }
      }
      a = pa[0];
      c = pc[0];
#pragma unroll
      for (int pp = 1; pp < TB_MAX_PARTS; ++pp) {
        if (pp < parts) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] += pa[pp][i];
            c[i] += pc[pp][i];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = c[i];
    }
  }
  float sc = 1.0f;
  if constexpr (XFORM) {
    fwht128_lanes(v, sub);
    sc = kInvSqrt128;
  }
  if constexpr (OUT == kOutAct8) {
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = f32_to_bf16_rne(v[e] * sc);
    // act8 buffer: values of block b at b * 512, scales at 4 * elements + b * 16
    uint8_t* act = static_cast<uint8_t*>(y);
    const int64_t bb = live ? b : 0;
    act8_encode_store(h, sub, act + bb * 512, act + nblocks * 512 + bb * 16, live);
    return;
  }
  if (!live) return;
  if constexpr (OUT == kOutBF16) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = f32_to_bf16_rne(v[2 * i] * sc) | (f32_to_bf16_rne(v[2 * i + 1] * sc) << 16);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + base) = w;
  } else {
    f32x4 a, c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = v[i] * sc;
      c[i] = v[4 + i] * sc;
    }
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(y) + base);
    p[0] = a;
    p[1] = c;
  }
}

__device__ __forceinline__ int wave_segment(const FwhtSegs& segs, int64_t bw) {
  // the wave's segment: the last whose first block is at or before bw
  int seg = 0;
#pragma unroll
  for (int t = 1; t < TB_MAX_SEGMENTS; ++t) seg += (t < segs.count && bw >= segs.s[t].begin) ? 1 : 0;
  return seg;
}

// every segment of the launch of one kind
template <bool IN_BF16, int OUT, bool XFORM>
__global__ void __launch_bounds__(64) fwht128_kernel(FwhtSegs segs) {
  const int sub = threadIdx.x & 15;
  for (int64_t bw = (int64_t)blockIdx.x * 4; bw < segs.total; bw += (int64_t)gridDim.x * 4) {
    const int seg = wave_segment(segs, bw);
    const int64_t b = bw - segs.s[seg].begin + (threadIdx.x >> 4);  // block inside its segment
    fwht_block<IN_BF16, OUT, XFORM>(segs.s[seg].x, segs.s[seg].y, segs.s[seg].nblocks, b, sub, segs.s[seg].parts);
  }
}

// segments of different kinds: the kind is uniform per wave, so the choice
// is a scalar branch
__global__ void __launch_bounds__(64) fwht128_mixed_kernel(FwhtSegs segs) {
  const int sub = threadIdx.x & 15;
  for (int64_t bw = (int64_t)blockIdx.x * 4; bw < segs.total; bw += (int64_t)gridDim.x * 4) {
    const int seg = wave_segment(segs, bw);
    const FwhtSeg& sg = segs.s[seg];
    const int64_t b = bw - sg.begin + (threadIdx.x >> 4);
    switch (__builtin_amdgcn_readfirstlane(sg.kind)) {
      case 0: fwht_block<false, kOutF32, true>(sg.x, sg.y, sg.nblocks, b, sub, sg.parts); break;
      case 1: fwht_block<false, kOutBF16, true>(sg.x, sg.y, sg.nblocks, b, sub, sg.parts); break;
      case 2: fwht_block<false, kOutAct8, true>(sg.x, sg.y, sg.nblocks, b, sub, sg.parts); break;
      case 3: fwht_block<true, kOutF32, true>(sg.x, sg.y, sg.nblocks, b, sub); break;
      case 4: fwht_block<true, kOutBF16, true>(sg.x, sg.y, sg.nblocks, b, sub); break;
      default: fwht_block<true, kOutAct8, true>(sg.x, sg.y, sg.nblocks, b, sub); break;
    }
  }
}

int seg_kind(int x_dtype, int y_dtype) {
  const int out = y_dtype == TB_ACT8 ? kOutAct8 : y_dtype == TB_BF16 ? kOutBF16 : kOutF32;
  return 3 * (x_dtype == TB_BF16 ? 1 : 0) + out;
}

unsigned grid_of(int64_t total) {
  const int64_t groups = (total + 3) / 4, cap = 1 << 20;
  return (unsigned)(groups < cap ? groups : cap);
}

template <bool XFORM>
hipError_t launch_segments(const FwhtSegs& segs, int x_dtype, int y_dtype, hipStream_t stream) {
  if (segs.total == 0) return hipSuccess;
  const dim3 g(grid_of(segs.total)), blk(64);
  const bool ib = x_dtype == TB_BF16;
  if (y_dtype == TB_ACT8) {
    if (ib) hipLaunchKernelGGL((fwht128_kernel<true, kOutAct8, XFORM>), g, blk, 0, stream, segs);
    else hipLaunchKernelGGL((fwht128_kernel<false, kOutAct8, XFORM>), g, blk, 0, stream, segs);
  } else if (y_dtype == TB_BF16) {
    if (ib) hipLaunchKernelGGL((fwht128_kernel<true, kOutBF16, XFORM>), g, blk, 0, stream, segs);
    else hipLaunchKernelGGL((fwht128_kernel<false, kOutBF16, XFORM>), g, blk, 0, stream, segs);
  } else {
    if (ib) hipLaunchKernelGGL((fwht128_kernel<true, kOutF32, XFORM>), g, blk, 0, stream, segs);
    else hipLaunchKernelGGL((fwht128_kernel<false, kOutF32, XFORM>), g, blk, 0, stream, segs);
  }
  return hipGetLastError();
}

FwhtSegs one_segment(const void* x, void* y, int64_t nblocks) {
  FwhtSegs s{};
  s.s[0] = FwhtSeg{x, y, nblocks, 0, 0, 1};
  s.count = 1;
  s.total = nblocks;
  return s;
}

}  // namespace

hipError_t launch_fwht128(const void* x, int x_dtype, void* y, int y_dtype, int64_t rows, int64_t K,
                          hipStream_t stream) {
  return launch_segments<true>(one_segment(x, y, rows * (K / kBlock)), x_dtype, y_dtype, stream);
}

hipError_t launch_fwht128_multi(const tb_fwht_segment* segs, int count, hipStream_t stream) {
  FwhtSegs s{};
  int64_t total = 0;
  bool same = true;
  for (int c = 0; c < count; ++c) {
    const int64_t nb = segs[c].rows * (segs[c].K / kBlock);
    s.s[c] = FwhtSeg{segs[c].x, segs[c].y, nb, total, seg_kind(segs[c].x_dtype, segs[c].y_dtype),
                     segs[c].x_parts > 1 ? segs[c].x_parts : 1};
    total += (nb + 3) / 4 * 4;  // the next segment starts on a wave boundary
    same = same && s.s[c].kind == s.s[0].kind;
  }
  s.count = count;
  s.total = total;
  if (count == 0) return hipSuccess;
  if (same) return launch_segments<true>(s, segs[0].x_dtype, segs[0].y_dtype, stream);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(fwht128_mixed_kernel, dim3(grid_of(total)), dim3(64), 0, stream, s);
  return hipGetLastError();
}

hipError_t launch_act8_prep(const uint16_t* x, int64_t rows, int64_t K, uint8_t* act, hipStream_t stream) {
  return launch_segments<false>(one_segment(x, act, rows * (K / kBlock)), TB_BF16, TB_ACT8, stream);
}

}  // namespace tb
