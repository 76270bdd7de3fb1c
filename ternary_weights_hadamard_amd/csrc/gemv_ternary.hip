// Decode GEMV with dense ternary weights:
//   y[b][n] = sum_g f16(scale[n][g]) * sum_{k in g} t[n][k] * x[b][k]
// (mhpq.cn/news/1159370 §4.2: read the weight bits, expand, scale, multiply).
//
// HBM bound: every weight is streamed once at 2 bits plus 1/8 bit of scale,
// so the kernel spends as little vector-ALU work per weight as possible and
// keeps as many code loads in flight as the registers allow.
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
// Work split: a wave owns one 16-row tile and a slice of at most CH groups of
// K; it issues every load of its slice (activations, codes and scales, group
// by group) before the first instruction that needs one, so all of them are in
// flight at once and the in-order load counter never makes a far load wait for
// a near one.  The KS slices of a tile are the waves of one workgroup and are
// added through LDS in a fixed order (the result does not depend on timing).
#include <algorithm>

#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kMaxSlices = 16;  // waves per workgroup
constexpr int kMaxSegs = TB_MAX_SEGMENTS;

// groups per wave and chunk: a group costs 9 * NB4 + 3 registers, and a
// workgroup of up to 16 waves leaves 128 per lane
template <int NB4>
struct Chunk {
  static constexpr int value = NB4 == 1 ? 9 : NB4 == 2 ? 4 : NB4 == 3 ? 3 : 2;
};

template <int NB4, int CH>
__global__ void __launch_bounds__(64 * kMaxSlices) gemv_direct_kernel(const uint8_t* __restrict__ act, int B,
                                                                        const uint32_t* __restrict__ codes,
                                                                        const uint16_t* __restrict__ scales,
                                                                        int64_t N, int64_t K, int P,
                                                                        float* __restrict__ y, int KS) {
  __shared__ float red[kMaxSlices][NB4][64];
  const int lane = threadIdx.x & 63;
  const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, q = lane >> 4;
  const int64_t nb = blockIdx.x;
  const int GA = (int)(K / kBlock);  // activation groups per row
  const int G = GA * P;              // code and scale groups per row (P planes)
  const int gb = G * ks / KS, ge = G * (ks + 1) / KS;

  // activation operand rows of this lane: batch 4m + i/4, sub-row i % 4
  const uint8_t* av_base[NB4];
  const uint8_t* as_base[NB4];
  bool arow[NB4];
#pragma unroll
  for (int m = 0; m < NB4; ++m) {
    const int b = 4 * m + (i >> 2);
    arow[m] = b < B;
    const size_t row = (size_t)(arow[m] ? b : 0) * GA;
    av_base[m] = act + (row * 16 + (i & 3) * 4 + q) * 32;
    as_base[m] = act + (size_t)4 * B * K + row * 16 + (i & 3) * 4 + q;
  }
  const uint32_t* cp = codes + (size_t)nb * G * 128 + 2 * lane;
  const uint16_t* sp = scales + (size_t)(16 * nb + i) * G;

  float acc[NB4];
#pragma unroll
  for (int m = 0; m < NB4; ++m) acc[m] = 0.f;

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  for (int c = gb; c < ge; c += CH) {
    const int n = min(CH, ge - c);
    i32x8 av[CH][NB4];
    int as[CH][NB4];
    u32x2 cw[CH];
    uint32_t sw[CH];
    // every load of the chunk first (slots past the slice repeat its last group;
    // the loops stay free of early exits so the arrays live in registers)
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int g = min(c + j, ge - 1);
      const int ga = P == 1 ? g : g >> 1;  // the activation group of code group g
      cw[j] = *reinterpret_cast<const u32x2*>(cp + (size_t)g * 128);
      sw[j] = sp[g];
#pragma unroll
      for (int m = 0; m < NB4; ++m) {
        if (arow[m]) {
          const u32x4* p = reinterpret_cast<const u32x4*>(av_base[m] + (size_t)ga * 512);
          const u32x4 lo = p[0], hi = p[1];
          av[j][m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          as[j][m] = as_base[m][(size_t)ga * 16];
        } else {
          av[j][m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
          as[j][m] = 127;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t w0 = cw[j][0], w1 = cw[j][1];
      const i32x4 bw = {(int)(w0 & 0xCCCCCCCCu), (int)((w0 << 2) & 0xCCCCCCCCu), (int)(w1 & 0xCCCCCCCCu),
                        (int)((w1 << 2) & 0xCCCCCCCCu)};
      const i32x8 b8 = {bw[0], bw[1], bw[2], bw[3], 0, 0, 0, 0};  // fp4 uses the low four registers
      const float s = f16_bits_to_f32(sw[j]) * 0.5f;
#pragma unroll
      for (int m = 0; m < NB4; ++m) {
        const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[j][m], b8, zero, 0, 4, 0, as[j][m], 0, 127);
        // the destination must not reuse the sources' registers (the
        // instruction reads them over several passes)
        keep_sources_past(d, av[j][m], bw);
        const float a = __builtin_fmaf(s, (d[0] + d[1]) + (d[2] + d[3]), acc[m]);
        acc[m] = j < n ? a : acc[m];  // slots past the slice (a repeated group) add nothing
      }
    }
  }

  if (KS > 1) {
#pragma unroll
    for (int m = 0; m < NB4; ++m) red[ks][m][lane] = acc[m];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int m = 0; m < NB4; ++m)
      for (int w = 1; w < KS; ++w) acc[m] += red[w][m][lane];
  }
#pragma unroll
  for (int m = 0; m < NB4; ++m) {
    const int b = 4 * m + q;
    if (b < B) y[(size_t)b * N + 16 * nb + i] = acc[m];
  }
}


// Staged path (B <= 4, the activation slices of a workgroup fit in LDS).  Per
// wave: the activation operand of its slice is copied into a private LDS area
// with whole-wave 16-byte loads (one load moves two groups of one batch row),
// the weight scales come in with one load per four groups (lane (i, q) fetches
// group 4r + q of row i) and are handed to the other lanes with ds_bpermute,
// and the codes with one load per group.  That is about CH + CH/2 + CH/4 + 1
// loads for CH groups instead of 5 CH, which matters because the number of
// loads a wave can keep in flight, not their size, bounds this kernel.
//
// One launch can carry up to kMaxSegs independent products (segments), e.g.
// the projections of one layer: workgroups are numbered across segments and
// each finds its own.  A segment splits K over ks waves (a power of two); a
// workgroup of `waves` waves covers waves / ks tiles of it.
constexpr int kStageBytes = 528;  // act8 bytes per group and batch row (512 values + 16 scales)
constexpr size_t kStagedMaxLds = 96 * 1024;
// groups per wave: 10 for one batch row, 8 when up to four rows are staged
// (the staging registers grow with the rows).  A batch-1 group whose longest
// K would need more than 8 waves per tile takes 18 groups per wave instead:
// 8-wave workgroups of at most 76 KB LDS, two per CU, rather than 16-wave
// ones that fit only once per CU.
constexpr int staged_ch(int bmax) { return bmax == 1 ? 10 : 8; }
constexpr int kLongCH = 18;

struct StagedSeg {
  const uint8_t* act;
  const uint32_t* codes;
  const uint16_t* scales;
  float* y;
  int64_t N, K;
  int B, ks, wg_begin, pad;
};

struct StagedSegs {
  StagedSeg s[kMaxSegs];
  int count, bmax;
  int stage_groups;  // activation groups staged per wave and batch row (two planes)
};

// the segment of this workgroup, selected field by field (the index is
// uniform, so these are scalar selects on kernel arguments)
__device__ __forceinline__ StagedSeg pick_segment(const StagedSegs& a) {
  const int wg = (int)blockIdx.x;
  StagedSeg r = a.s[0];
#pragma unroll
  for (int t = 1; t < kMaxSegs; ++t) {
    const bool take = t < a.count && wg >= a.s[t].wg_begin;
    r.act = take ? a.s[t].act : r.act;
    r.codes = take ? a.s[t].codes : r.codes;
    r.scales = take ? a.s[t].scales : r.scales;
    r.y = take ? a.s[t].y : r.y;
    r.N = take ? a.s[t].N : r.N;
    r.K = take ? a.s[t].K : r.K;
    r.B = take ? a.s[t].B : r.B;
    r.ks = take ? a.s[t].ks : r.ks;
    r.wg_begin = take ? a.s[t].wg_begin : r.wg_begin;
  }
  return r;
}

// P code planes per segment (1, or 2 with the planes' groups interleaved)
template <int CH, int BMAX, int P>
__global__ void __launch_bounds__(64 * kMaxSlices) gemv_staged_kernel(StagedSegs segs) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const StagedSeg sg = pick_segment(segs);
  const uint8_t* __restrict__ act = sg.act;
  const int B = sg.B, KS = sg.ks;
  const int64_t N = sg.N, K = sg.K;
  const int waves = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ks = w % KS;
  const int i = lane & 15, q = lane >> 4;
  const int64_t nb = (int64_t)(blockIdx.x - sg.wg_begin) * (waves / KS) + w / KS;
  const bool live = nb < N / 16;
  const int GA = (int)(K / kBlock);  // activation groups per row
  const int G = GA * P;              // code and scale groups per row
  const int gb = G * ks / KS, ge = G * (ks + 1) / KS;
  const int n = ge - gb;  // 1 .. CH code groups in this slice
  // activation groups of the slice: code group g multiplies activation group g / P
  const int ab = gb / P, na = (ge - 1) / P - ab + 1;
  constexpr int kPairs = (CH + 1) / 2;
  constexpr int kScaleRegs = (CH + 3) / 4;
  const int SG = P == 1 ? CH : segs.stage_groups;  // >= na
  const size_t region = (size_t)segs.bmax * SG * kStageBytes;
  unsigned char* st = smem + (size_t)w * region;  // [B][SG][512] values, then [B][SG][16] scales
  unsigned char* st_sc = st + (size_t)B * SG * 512;
  float* red = reinterpret_cast<float*>(smem + (size_t)waves * region);

  float acc = 0.f;
  if (live) {
    // 1. activation slice (issued first: it is waited for first)
    u32x4 av_st[BMAX][kPairs];
    u32x4 as_st[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      const unsigned char* src = act + ((size_t)b * GA + ab) * 512;
#pragma unroll
      for (int t = 0; t < kPairs; ++t) {
        const int off = t * 1024 + lane * 16;
        if (b < B && off < na * 512) av_st[b][t] = *reinterpret_cast<const u32x4*>(src + off);
      }
      if (b < B && lane < na)
        as_st[b] = *reinterpret_cast<const u32x4*>(act + (size_t)4 * B * K + ((size_t)b * GA + ab + lane) * 16);
    }
    // 2. codes, one 8-byte load per lane and group (slots past the slice repeat its last group)
    const uint32_t* cp = sg.codes + (size_t)nb * G * 128 + 2 * lane;
    u32x2 cw[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) cw[j] = *reinterpret_cast<const u32x2*>(cp + (size_t)min(gb + j, ge - 1) * 128);
    // 3. weight scales: lane (i, q) holds row i's scale of groups gb + 4r + q
    const uint16_t* sp = sg.scales + (size_t)(16 * nb + i) * G;
    uint32_t sr[kScaleRegs];
#pragma unroll
    for (int r = 0; r < kScaleRegs; ++r) sr[r] = sp[min(gb + 4 * r + q, ge - 1)];
    // 4. activation slice into this wave's LDS area (read back by other lanes of
    //    the same wave only; LDS operations of a wave complete in order)
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
#pragma unroll
      for (int t = 0; t < kPairs; ++t) {
        const int off = t * 1024 + lane * 16;
        if (b < B && off < na * 512) *reinterpret_cast<u32x4*>(st + (size_t)b * SG * 512 + off) = av_st[b][t];
      }
      if (b < B && lane < na) *reinterpret_cast<u32x4*>(st_sc + ((size_t)b * SG + lane) * 16) = as_st[b];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // 5. the products: lane (i, q) feeds A rows of batch i / 4, sub-row i % 4.
    //    Rows of batches >= B only reach output rows that are never stored, so
    //    those lanes read the last batch row instead of branching.
    const int bp = min(i >> 2, B - 1);
    const unsigned char* a_src = st + (size_t)bp * SG * 512 + ((i & 3) * 4 + q) * 32;
    const unsigned char* a_sc = st_sc + (size_t)bp * SG * 16 + (i & 3) * 4 + q;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      // staged activation group of slot j (slots past the slice repeat the last one)
      const int aj = P == 1 ? j : (min(gb + j, ge - 1) >> 1) - ab;
      const u32x4* p = reinterpret_cast<const u32x4*>(a_src + aj * 512);
      const u32x4 lo = p[0], hi = p[1];
      const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      const int as = a_sc[aj * 16];
      const int sbits = __builtin_amdgcn_ds_bpermute((i + 16 * (j & 3)) * 4, (int)sr[j >> 2]);
      const float s = f16_bits_to_f32((uint32_t)sbits & 0xFFFFu) * 0.5f;
      const uint32_t w0 = cw[j][0], w1 = cw[j][1];
      const i32x4 bw = {(int)(w0 & 0xCCCCCCCCu), (int)((w0 << 2) & 0xCCCCCCCCu), (int)(w1 & 0xCCCCCCCCu),
                        (int)((w1 << 2) & 0xCCCCCCCCu)};
      const i32x8 b8 = {bw[0], bw[1], bw[2], bw[3], 0, 0, 0, 0};  // fp4 uses the low four registers
      const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b8, zero, 0, 4, 0, as, 0, 127);
      keep_sources_past(d, av, bw);  // the destination must not reuse the sources' registers
      const float a = __builtin_fmaf(s, (d[0] + d[1]) + (d[2] + d[3]), acc);
      acc = j < n ? a : acc;  // slots past the slice add nothing
    }
  }

  if (KS > 1) {
    red[w * 64 + lane] = acc;
    __syncthreads();
    if (ks != 0) return;
    for (int u = 1; u < KS; ++u) acc += red[(w + u) * 64 + lane];
  }
  if (live && q < B) sg.y[(size_t)q * N + 16 * nb + i] = acc;
}

int slices(int64_t K, int ch) {
  const int64_t G = K / kBlock;
  return (int)std::min<int64_t>(kMaxSlices, (G + ch - 1) / ch);
}

// K slices of a staged segment: the smallest power of two giving at most ch
// groups per wave, or 0 when even kMaxSlices waves are too few
int staged_slices(int64_t K, int ch) {
  const int64_t G = K / kBlock;
  for (int ks = 1; ks <= kMaxSlices; ks *= 2)
    if (G <= (int64_t)ks * ch) return ks;
  return 0;
}

}  // namespace

// Groups per wave of one segment, a function of its own code length K (all
// planes) and B only, so that a segment is cut into the same K slices (and
// summed in the same order) whatever it is launched with.
int segment_ch(int64_t K, int64_t B) {
  if (B > 1) return staged_ch(4);
  const int ks = staged_slices(K, staged_ch(1));
  return ks != 0 && ks <= 8 ? staged_ch(1) : kLongCH;
}

hipError_t launch_gemv_multi(const GemvSegment* segs, int count, hipStream_t stream) {
  // one grouped launch when every segment fits the staged path together, else
  // each segment on its own exactly as a single call would run it
  StagedSegs st{};
  bool staged = count <= kMaxSegs;
  int bmax = 1, ch = 1, waves = 1, wg = 0;
  const int64_t planes = count > 0 ? segs[0].planes : 1;
  for (int c = 0; c < count && staged; ++c) {
    const int64_t kc = segs[c].K * segs[c].planes;  // code groups x 128
    const int sc = segment_ch(kc, segs[c].B);
    const int ks = staged_slices(kc, sc);
    if (segs[c].B > 4 || ks == 0) staged = false;
    bmax = std::max(bmax, (int)segs[c].B);
    ch = std::max(ch, sc);
    waves = std::max(waves, ks);
    if (segs[c].planes != planes) staged = false;  // one plane count per grouped launch
  }
  // kernels exist for (10, 1), (18, 1) and (8, up to 4 rows)
  if (bmax > 1 && ch != staged_ch(4)) staged = false;
  // a slice of at most ch code groups spans at most ch activation groups with
  // one plane, ch / 2 + 1 with two
  const int stage_groups = planes == 1 ? ch : ch / 2 + 1;
  const size_t lds = (size_t)waves * bmax * stage_groups * kStageBytes + (size_t)waves * 64 * sizeof(float);
  if (staged && lds <= kStagedMaxLds) {
    for (int c = 0; c < count; ++c) {
      const int64_t kc = segs[c].K * segs[c].planes;
      const int ks = staged_slices(kc, segment_ch(kc, segs[c].B));
      const int64_t tiles = segs[c].N / 16, per_wg = waves / ks;
      st.s[c] = StagedSeg{segs[c].act, segs[c].codes, segs[c].scales, segs[c].y, segs[c].N, segs[c].K,
                          (int)segs[c].B, ks, wg, 0};
      wg += (int)((tiles + per_wg - 1) / per_wg);
    }
    st.count = count;
    st.bmax = bmax;
    st.stage_groups = stage_groups;
    const dim3 grid((unsigned)wg), block(64 * waves);
#define TB_STAGED(CH_, BMAX_, P_) hipLaunchKernelGGL((gemv_staged_kernel<CH_, BMAX_, P_>), grid, block, lds, stream, st)
    if (planes == 1) {
      if (bmax == 1 && ch == kLongCH)
        TB_STAGED(kLongCH, 1, 1);
      else if (bmax == 1)
        TB_STAGED(staged_ch(1), 1, 1);
      else
        TB_STAGED(staged_ch(4), 4, 1);
    } else {
      if (bmax == 1 && ch == kLongCH)
        TB_STAGED(kLongCH, 1, 2);
      else if (bmax == 1)
        TB_STAGED(staged_ch(1), 1, 2);
      else
        TB_STAGED(staged_ch(4), 4, 2);
    }
#undef TB_STAGED
    return hipGetLastError();
  }
  if (count == 1)
    return launch_gemv_direct(segs[0].act, segs[0].B, segs[0].codes, segs[0].scales, segs[0].N, segs[0].K,
                              (int)segs[0].planes, segs[0].y, stream);
  for (int c = 0; c < count; ++c) {
    const hipError_t e = launch_gemv_multi(segs + c, 1, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemv_direct(const uint8_t* act, int64_t B, const uint32_t* codes, const uint16_t* scales,
                              int64_t N, int64_t K, int planes, float* y, hipStream_t stream) {
  const dim3 grid((unsigned)(N / 16));
  const int b = (int)B;
  switch ((B + 3) / 4) {
    case 1: {
      const int ks = slices(K * planes, Chunk<1>::value);
      hipLaunchKernelGGL((gemv_direct_kernel<1, Chunk<1>::value>), grid, dim3(64 * ks), 0, stream, act, b, codes,
                         scales, N, K, planes, y, ks);
      break;
    }
    case 2: {
      const int ks = slices(K * planes, Chunk<2>::value);
      hipLaunchKernelGGL((gemv_direct_kernel<2, Chunk<2>::value>), grid, dim3(64 * ks), 0, stream, act, b, codes,
                         scales, N, K, planes, y, ks);
      break;
    }
    case 3: {
      const int ks = slices(K * planes, Chunk<3>::value);
      hipLaunchKernelGGL((gemv_direct_kernel<3, Chunk<3>::value>), grid, dim3(64 * ks), 0, stream, act, b, codes,
                         scales, N, K, planes, y, ks);
      break;
    }
    default: {
      const int ks = slices(K * planes, Chunk<4>::value);
      hipLaunchKernelGGL((gemv_direct_kernel<4, Chunk<4>::value>), grid, dim3(64 * ks), 0, stream, act, b, codes,
                         scales, N, K, planes, y, ks);
      break;
    }
  }
  return hipGetLastError();
}


}  // namespace tb
