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
// Two kernels split the work:
//   * batch 1 (staged): a wave owns one or two 16-row tiles and a slice of K,
//     stages its activation slice in LDS and issues every load of the slice
//     before the first instruction that needs one;
//   * batch 2-16, and batch 1 past the staged slices (wide): a wave owns T
//     consecutive tiles and a slice of K, walked
//     in chunks, and applies each activation fragment to all T tiles.
// The K slices of a tile are waves of one workgroup and are added through LDS
// in a fixed order, so a result does not depend on timing or on which
// segments share its launch.
#include <algorithm>

#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kMaxSlices = 16;  // waves per workgroup
constexpr int kMaxSegs = TB_MAX_SEGMENTS;

// Staged path (batch 1, the activation slices of a workgroup fit in LDS).  Per
// wave: the activation operand of its slice is copied into a private LDS area
// with whole-wave 16-byte loads (one load moves two groups of one batch row),
// the weight scales come in with one load per eight groups of its tile and
// are handed to the other lanes with ds_bpermute, and the codes with one load
// per group.  That is about CH + CH/2 + CH/8 + 1 loads for CH groups instead of
// 5 CH, which matters because the number of loads a wave can keep in flight,
// not their size, bounds this kernel.  A wave may take two consecutive tiles
// at its K slice, which share the staged activations.
//
// One launch can carry up to kMaxSegs independent products (segments), e.g.
// the projections of one layer: workgroups are numbered across segments and
// each finds its own.  A segment splits K over ks waves (a power of two); a
// workgroup of `waves` waves covers waves / ks tiles of it.
constexpr int kStageBytes = 528;  // act8 bytes per group and batch row (512 values + 16 scales)
constexpr size_t kStagedMaxLds = 96 * 1024;
// groups per wave: 10.  A group whose longest K would need more than 8 waves
// per tile takes 17 groups per wave instead: 8-wave workgroups of at most 72 KB
// LDS, two per CU, rather than 16-wave ones that fit only once per CU.  17 is
// the slice of a 17408-long K (136 groups = 8 x 17) with no repeated slot
// (1.5 % faster than 18 on the 27B down projection).
constexpr int kStagedCH = 10;
constexpr int kLongCH = 17;
constexpr int64_t kTwoTileMin = 2048;  // tiles in a launch before a wave takes two

struct StagedSeg {
  const uint8_t* act;
  const uint32_t* codes;
  const uint16_t* scales;
  float* y;
  int64_t N, K;
  int B, ks, wg_begin;
  int lgp;  // log2 of the segment's K parts: workgroups per tile, each writing its part of y
};

struct StagedSegs {
  StagedSeg s[kMaxSegs];
  int count, bmax;
  int stage_groups;  // activation groups staged per wave and batch row (two planes)
};

// the segment of this workgroup: its index from the workgroup starts, then
// that one entry's fields (a uniform index, so scalar loads of the kernel
// arguments; selecting every field across all entries kept them all live
// and spilled scalar registers)
template <class Segs>
__device__ __forceinline__ int segment_index(const Segs& a) {
  const int wg = (int)blockIdx.x;
  int seg = 0;
#pragma unroll
  for (int t = 1; t < kMaxSegs; ++t) seg += (t < a.count && wg >= a.s[t].wg_begin) ? 1 : 0;
  return seg;
}

// Entry 0 is read alongside the workgroup starts, so that the workgroups of
// the first segment (all of them in a one-segment launch) do not wait for a
// second round of scalar loads.
__device__ __forceinline__ StagedSeg pick_segment(const StagedSegs& a) {
  const StagedSeg r0 = a.s[0];
  const int seg = segment_index(a);
  return seg == 0 ? r0 : a.s[seg];
}

// P code planes per segment (1, or 2 with the planes' groups interleaved); T
// consecutive tiles per wave at the same K slice, which share the staged
// activation slice
template <int CH, int BMAX, int P, int T>
__global__ void __launch_bounds__(64 * kMaxSlices) gemv_staged_kernel(StagedSegs segs) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const StagedSeg sg = pick_segment(segs);
  const uint8_t* __restrict__ act = sg.act;
  const int B = sg.B, KS = sg.ks;  // K slices of a tile, over all its parts
  const int64_t N = sg.N, K = sg.K;
  const int waves = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // KS, the parts and waves are powers of two (waves the largest slices per
  // part of the launch), so the slice arithmetic is shifts and masks: a wave
  // starts its loads sooner.  A tile's parts are consecutive workgroups; part
  // p adds slices [p KSW, (p + 1) KSW), KSW = KS / parts, one per wave.
  const int lg = __builtin_ctz((unsigned)KS);
  const int lgp = sg.lgp, lgw = lg - lgp;
  const int64_t wgl = (int64_t)(blockIdx.x - sg.wg_begin);
  const int part = (int)(wgl & ((1 << lgp) - 1));
  const int ksw = w & ((1 << lgw) - 1);
  const int ks = (part << lgw) + ksw;
  const int i = lane & 15, q = lane >> 4;
  const int64_t nb0 = ((wgl >> lgp) * (waves >> lgw) + (w >> lgw)) * T;
  const int64_t ntiles = (int64_t)((uint64_t)N >> 4);
  const bool live = nb0 < ntiles;
  const int GA = (int)((uint64_t)K >> 7);  // activation groups per row
  const int G = GA * P;                    // code and scale groups per row
  const int gb = (G * ks) >> lg, ge = (G * (ks + 1)) >> lg;
  const int n = ge - gb;  // 1 .. CH code groups in this slice
  // activation groups of the slice: code group g multiplies activation group g / P
  const int ab = gb / P, na = (ge - 1) / P - ab + 1;
  constexpr int kPairs = (CH + 1) / 2;
  const int SG = P == 1 ? CH : segs.stage_groups;  // >= na
  const size_t region = (size_t)segs.bmax * SG * kStageBytes;
  unsigned char* st = smem + (size_t)w * region;  // [B][SG][512] values, then [B][SG][16] scales
  unsigned char* st_sc = st + (size_t)B * SG * 512;
  float* red = reinterpret_cast<float*>(smem + (size_t)waves * region);

  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.f;
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
    // 2. weight scales, issued before the codes so that each product waits
    //    only for its own code group (a 27B layer's down projection at batch
    //    1: 12.2 -> 11.9 us).  Scales are tile-major, [N/16][G][16], so one
    //    dword load brings 8 groups of the tile (lane l: group gb + 8 r + l / 8,
    //    rows 2 (l % 8) and 2 (l % 8) + 1) from 256 contiguous bytes; with
    //    scales by row, each load of 16 rows touched 10-16 cache lines (a 27B
    //    layer at batch 1: 17.9 -> 16.4 us and 10.7 -> 9.7 us per launch).
    // 3. codes, one 8-byte load per lane and group (slots past the slice repeat
    //    its last group).  Non-temporal: read once, they need not displace the
    //    activations from the caches (batch 1 on a 27B layer's QKV + O +
    //    gate/up: 20.1 -> 19.45 us; down 12.6 -> 12.4 us)
    constexpr int kSR = (CH + 7) / 8;
    uint32_t sr[T][kSR];
    u32x2 cw[T][CH];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t nb = min(nb0 + t, ntiles - 1);  // tiles past the end repeat the last (never stored)
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(sg.scales + (size_t)nb * G * 16);
#pragma unroll
      for (int r = 0; r < kSR; ++r) sr[t][r] = sp[min((gb + 8 * r) * 8 + lane, ge * 8 - 1)];
      const uint32_t* cp = sg.codes + (size_t)nb * G * 128 + 2 * lane;
#pragma unroll
      for (int j = 0; j < CH; ++j)
        cw[t][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(cp + (size_t)min(gb + j, ge - 1) * 128));
    }
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
    //    those lanes read the last batch row instead of branching.  The scale
    //    of row i and group gb + j sits in lane 8 (j % 8) + i / 2, half i % 2.
    const int bp = min(i >> 2, B - 1);
    const unsigned char* a_src = st + (size_t)bp * SG * 512 + ((i & 3) * 4 + q) * 16;
    const unsigned char* a_sc = st_sc + (size_t)bp * SG * 16 + (i & 3) * 4 + q;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const int e8m0_one = 127;  // the weights' block scale: 2^0
    // The products are software-pipelined over a ring of three register sets:
    // step j's staged activations, activation scale and weight scale are read
    // from LDS into set j % 3 one step ahead, step j's product is issued while
    // step j - 1's may still run, and step j - 2's result is added before set
    // (j + 1) % 3 is refilled.  The sources of a product stay live (empty asm
    // uses) until its result has been read: otherwise the register allocator
    // may hand them to the next LDS reads while the product still reads them,
    // which gave wrong results.  The sum runs in step order as before, so the
    // result is unchanged (a 27B layer at batch 1: QKV + O + gate/up 16.0 ->
    // 15.3 us, down 9.75 -> 9.1 us per launch).
    struct Frag {
      u32x4 lo, hi;  // activation operand: sub-row values of the step's group
      int as;        // its E8M0 block scale
      int sb;        // two weight scales (fp16 bits), from ds_bpermute
    };
    auto fetch = [&](int t, int j, Frag& f) {
      // staged activation group of slot j (slots past the slice repeat the last one)
      const int aj = P == 1 ? j : (min(gb + j, ge - 1) >> 1) - ab;
      f.lo = *reinterpret_cast<const u32x4*>(a_src + aj * 512);
      f.hi = *reinterpret_cast<const u32x4*>(a_src + aj * 512 + 256);
      f.as = a_sc[aj * 16];
      f.sb = __builtin_amdgcn_ds_bpermute(((j & 7) * 8 + (i >> 1)) * 4, (int)sr[t][j >> 3]);
    };
#pragma unroll
    for (int t = 0; t < T; ++t) {
      Frag fr[3];
      f32x4 dd[3];
      i32x4 bws[3];
      auto add_step = [&](int j) {
        const Frag& g = fr[j % 3];
        const float s = f16_bits_to_f32(((uint32_t)g.sb >> ((i & 1) * 16)) & 0xFFFFu) * 0.5f;
        const f32x4 d = dd[j % 3];
        const float a = __builtin_fmaf(s, (d[0] + d[1]) + (d[2] + d[3]), acc[t]);
        acc[t] = j < n ? a : acc[t];  // slots past the slice add nothing
        const i32x8 av = {(int)g.lo[0], (int)g.lo[1], (int)g.lo[2], (int)g.lo[3],
                          (int)g.hi[0], (int)g.hi[1], (int)g.hi[2], (int)g.hi[3]};
        asm volatile("" ::"v"(av), "v"(bws[j % 3]), "v"(g.as), "v"(acc[t]));
      };
      fetch(t, 0, fr[0]);
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        if (j >= 2) add_step(j - 2);
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < CH) fetch(t, j + 1, fr[(j + 1) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        const Frag& f = fr[j % 3];
        const i32x8 av = {(int)f.lo[0], (int)f.lo[1], (int)f.lo[2], (int)f.lo[3],
                          (int)f.hi[0], (int)f.hi[1], (int)f.hi[2], (int)f.hi[3]};
        const uint32_t w0 = cw[t][j][0], w1 = cw[t][j][1];
        bws[j % 3] = i32x4{(int)(w0 & 0xCCCCCCCCu), (int)((w0 << 2) & 0xCCCCCCCCu), (int)(w1 & 0xCCCCCCCCu),
                           (int)((w1 << 2) & 0xCCCCCCCCu)};
        const i32x4 bw = bws[j % 3];
        const i32x8 b8 = {bw[0], bw[1], bw[2], bw[3], 0, 0, 0, 0};  // fp4 uses the low four registers
        dd[j % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b8, zero, 0, 4, 0, f.as, 0, e8m0_one);
        keep_sources_past(dd[j % 3], av, bw);  // the destination must not reuse the sources' registers
        asm volatile("" ::"v"(dd[j % 3]), "v"(f.as), "v"(e8m0_one));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (CH >= 2) add_step(CH - 2);
      add_step(CH - 1);
    }
  }

  if (lgw > 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) red[(w * T + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (ksw != 0) return;
#pragma unroll
    for (int t = 0; t < T; ++t)
      for (int u = 1; u < (1 << lgw); ++u) acc[t] += red[((w + u) * T + t) * 64 + lane];
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
    if (nb0 + t < ntiles && q < B) sg.y[((size_t)part * B + q) * N + 16 * (nb0 + t) + i] = acc[t];
}

// Wide path (B > 4, or a K too long for the staged slices).  A batch quad's
// activation operand is 8 registers (32 bytes) per lane and group, so at batch
// 8 one group of activations is eight times the bytes of one 16-row code
// tile; read once per tile, the activations would cost more cache-to-CU
// traffic than the codes cost HBM traffic.  A wave here covers T consecutive
// tiles of 16 output rows and applies each activation fragment to all of
// them.  The slice of K is walked in chunks of CH groups, every load of a
// chunk issued before its first product; per tile and chunk one scale load
// brings CH groups (lane (i, q) fetches row i's scale of group c + q) and
// ds_bpermute hands them to the other lanes.  Rows of batches >= B in the last
// quad read batch row B - 1 instead: a row of the instruction's A operand
// reaches only its own output row, which is never stored.  As in the staged
// path one launch carries several segments, a segment splits K over ks waves
// (a power of two) and the slices of a tile are added through LDS in a fixed
// order.  N is a multiple of 128, so a tile count is a multiple of 8 and a
// wave's T tiles (T divides 8) lie inside the segment or wholly past it.
struct WideSeg {
  const uint8_t* act;
  const uint32_t* codes;
  const uint16_t* scales;
  float* y;
  int64_t N, K;
  int B, P, ks, wg_begin;
  int lgp;  // log2 of the segment's K parts (as in the staged kernel)
};

struct WideSegs {
  WideSeg s[kMaxSegs];
  int count;
};

__device__ __forceinline__ WideSeg pick_wide_segment(const WideSegs& a) {
  const WideSeg r0 = a.s[0];
  const int seg = segment_index(a);
  return seg == 0 ? r0 : a.s[seg];
}

template <int NB4, int T, int CH>
__global__ void __launch_bounds__(64 * kMaxSlices) gemv_wide_kernel(WideSegs segs) {
  static_assert(8 % T == 0 && CH <= 4, "tile sets must divide 8 tiles; one scale load covers at most 4 groups");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const WideSeg sg = pick_wide_segment(segs);
  const int B = sg.B, KS = sg.ks, P = sg.P;
  const int64_t N = sg.N, K = sg.K;
  const int waves = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // KS, the parts and waves are powers of two: shifts and masks, and a tile
  // set's parts are consecutive workgroups, as in the staged kernel
  const int lg = __builtin_ctz((unsigned)KS);
  const int lgp = sg.lgp, lgw = lg - lgp;
  const int64_t wgl = (int64_t)(blockIdx.x - sg.wg_begin);
  const int part = (int)(wgl & ((1 << lgp) - 1));
  const int ksw = w & ((1 << lgw) - 1);
  const int ks = (part << lgw) + ksw;
  const int i = lane & 15, q = lane >> 4;
  const int64_t tiles = (int64_t)((uint64_t)N >> 4);
  const int64_t t0 = ((wgl >> lgp) * (waves >> lgw) + (w >> lgw)) * T;  // first tile
  const bool live = t0 < tiles;
  const int GA = (int)((uint64_t)K >> 7);  // activation groups per row
  const int G = GA * P;                    // code and scale groups per row
  const int gb = (G * ks) >> lg, ge = (G * (ks + 1)) >> lg;

  float acc[T][NB4];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int m = 0; m < NB4; ++m) acc[t][m] = 0.f;

  if (live) {
    // Addresses are a uniform base plus a 32-bit per-lane byte offset.
    // Activation operand rows of this lane: batch 4m + i / 4 (clamped to
    // B - 1), sub-row i % 4, lane group q.
    const unsigned char* act = sg.act;
    const unsigned char* act_sc = sg.act + (size_t)4 * B * K;
    uint32_t av_off[NB4], as_off[NB4];
#pragma unroll
    for (int m = 0; m < NB4; ++m) {
      const int b = min(4 * m + (i >> 2), B - 1);
      av_off[m] = (uint32_t)b * GA * 512 + ((i & 3) * 4 + q) * 16;
      as_off[m] = (uint32_t)b * GA * 16 + (i & 3) * 4 + q;
    }
    const unsigned char* cbase = reinterpret_cast<const unsigned char*>(sg.codes + (size_t)t0 * G * 128);
    const unsigned char* sbase = reinterpret_cast<const unsigned char*>(sg.scales + (size_t)16 * t0 * G);
    const uint32_t c_stride = (uint32_t)G * 512, s_stride = (uint32_t)G * 32;  // bytes per tile
    // scales [N/16][G][16]: lane (i, q) reads row i of group c + q, 32 bytes per group
    const uint32_t c_lane = (uint32_t)lane * 8, s_lane = (uint32_t)i * 2;

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int c = gb; c < ge; c += CH) {
      const int n = min(CH, ge - c);
      i32x8 av[CH][NB4];
      int as[CH][NB4];
      u32x2 cw[CH][T];
      uint32_t sr[T];
      // every load of the chunk first (slots past the slice repeat its last group)
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int g = min(c + j, ge - 1);
        const uint32_t ga = P == 1 ? g : g >> 1;  // the activation group of code group g
#pragma unroll
        for (int m = 0; m < NB4; ++m) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(act + (av_off[m] + ga * 512));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(act + (av_off[m] + ga * 512 + 256));
          av[j][m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          as[j][m] = act_sc[as_off[m] + ga * 16];
        }
#pragma unroll
        for (int t = 0; t < T; ++t)
          cw[j][t] = *reinterpret_cast<const u32x2*>(cbase + (t * c_stride + (uint32_t)g * 512 + c_lane));
      }
      const uint32_t gq = (uint32_t)min(c + q, ge - 1);
#pragma unroll
      for (int t = 0; t < T; ++t)
        sr[t] = *reinterpret_cast<const uint16_t*>(sbase + (t * s_stride + s_lane + gq * 32));
#pragma unroll
      for (int j = 0; j < CH; ++j) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t w0 = cw[j][t][0], w1 = cw[j][t][1];
          const i32x4 bw = {(int)(w0 & 0xCCCCCCCCu), (int)((w0 << 2) & 0xCCCCCCCCu), (int)(w1 & 0xCCCCCCCCu),
                            (int)((w1 << 2) & 0xCCCCCCCCu)};
          const i32x8 b8 = {bw[0], bw[1], bw[2], bw[3], 0, 0, 0, 0};  // fp4 uses the low four registers
          const int sbits = __builtin_amdgcn_ds_bpermute((i + 16 * j) * 4, (int)sr[t]);
          const float s = f16_bits_to_f32((uint32_t)sbits & 0xFFFFu) * 0.5f;
#pragma unroll
          for (int m = 0; m < NB4; ++m) {
            const f32x4 d =
                __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[j][m], b8, zero, 0, 4, 0, as[j][m], 0, 127);
            keep_sources_past(d, av[j][m], bw);  // the destination must not reuse the sources' registers
            const float a = __builtin_fmaf(s, (d[0] + d[1]) + (d[2] + d[3]), acc[t][m]);
            acc[t][m] = j < n ? a : acc[t][m];  // slots past the slice add nothing
          }
        }
      }
    }
  }

  if (lgw > 0) {
    float* red = reinterpret_cast<float*>(smem);  // [waves][T][NB4][64]
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int m = 0; m < NB4; ++m) red[((w * T + t) * NB4 + m) * 64 + lane] = acc[t][m];
    __syncthreads();
    if (ksw != 0) return;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int m = 0; m < NB4; ++m)
        for (int u = 1; u < (1 << lgw); ++u) acc[t][m] += red[(((w + u) * T + t) * NB4 + m) * 64 + lane];
  }
  if (live) {
    float* yp = sg.y + (size_t)part * B * N;
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int m = 0; m < NB4; ++m) {
        const int b = 4 * m + q;
        if (b < B) yp[(size_t)b * N + 16 * (t0 + t) + i] = acc[t][m];
      }
    }
  }
}

// Groups per chunk of the wide path: a group costs 9 * NB4 + 2 * T registers
// per lane, and T * NB4 accumulators stay live.  Above batch 8 one group per
// chunk keeps the registers low enough for more waves (batch 16 on a 27B
// layer's QKV + O + gate/up: 59.6 against 68.6 us); below it, longer chunks win.
template <int NB4, int T>
struct WideChunk {
  static constexpr int value = NB4 >= 3 ? 1 : NB4 * 9 + 2 * T <= 26 ? 3 : 2;
};

// K slices of a wide segment: the smallest power of two leaving at most
// kWideSlice groups per wave
constexpr int kWideSlice = 6;
int wide_slices(int64_t G) {
  int ks = 1;
  while (ks < kMaxSlices && G > (int64_t)ks * kWideSlice) ks *= 2;
  return ks;
}

// K slices of a staged segment: the smallest power of two giving at most ch
// groups per wave, or 0 when even max_ks slices are too few (a tile's slices
// are the waves of one workgroup, or of `parts` workgroups)
int staged_slices(int64_t K, int ch, int max_ks = kMaxSlices) {
  const int64_t G = K / kBlock;
  for (int ks = 1; ks <= max_ks; ks *= 2)
    if (G <= (int64_t)ks * ch) return ks;
  return 0;
}

}  // namespace

// Groups per wave of one staged segment, a function of its own code length K
// (all planes) only, so that a segment is cut into the same K slices (and
// summed in the same order) whatever it is launched with.
int segment_ch(int64_t K) {
  const int ks = staged_slices(K, kStagedCH);
  return ks != 0 && ks <= 8 ? kStagedCH : kLongCH;
}

// K slices of a staged segment's tiles (over all its parts) and its groups per
// wave.  A segment split into parts takes the short slices (at most
// kStagedCH groups), at least one slice per part and at most kMaxSlices per
// part (the waves of one workgroup).
void staged_geometry(const GemvSegment& g, int& ks, int& ch) {
  const int64_t kc = g.K * g.planes;  // code groups x 128
  if (g.parts > 1) {
    ch = kStagedCH;
    ks = std::max(staged_slices(kc, ch, kMaxSlices * (int)g.parts), (int)g.parts);
  } else {
    ch = segment_ch(kc);
    ks = staged_slices(kc, ch);
  }
}

// The staged path takes a batch-1 segment whose K fits the staged slices;
// everything else takes the wide path (from batch 2 on it is the faster one:
// 27 against 40 us at batch 2 on a 27B layer's QKV + O + gate/up).
bool stageable(const GemvSegment& g) {
  const int64_t kc = g.K * g.planes;  // code groups x 128
  return g.B == 1 && staged_slices(kc, segment_ch(kc)) != 0;
}

// Wide launch geometry for T tiles per wave: workgroups, waves per workgroup
// and the segment table
// K slices of a wide segment's tiles over all its parts: at least one per part
int wide_segment_slices(const GemvSegment& g) {
  return std::max(wide_slices(g.K / kBlock * g.planes), (int)g.parts);
}

int wide_plan(const GemvSegment* segs, int count, int T, WideSegs& ws, int& waves) {
  waves = 1;
  for (int c = 0; c < count; ++c) waves = std::max(waves, wide_segment_slices(segs[c]) / (int)segs[c].parts);
  int wg = 0;
  for (int c = 0; c < count; ++c) {
    const int ks = wide_segment_slices(segs[c]), parts = (int)segs[c].parts;
    const int64_t sets = segs[c].N / 16 / T, per_wg = waves / (ks / parts);
    ws.s[c] = WideSeg{segs[c].act, segs[c].codes, segs[c].scales, segs[c].y, segs[c].N, segs[c].K,
                      (int)segs[c].B, (int)segs[c].planes, ks, wg, __builtin_ctz((unsigned)parts)};
    wg += (int)((sets + per_wg - 1) / per_wg * parts);
  }
  ws.count = count;
  return wg;
}

constexpr int kWideTMax = 8;         // tiles per wave, at most
constexpr int kWideMinWaves = 2048;  // waves a launch should have before T is lowered

template <int NB4, int T>
hipError_t launch_wide_t(const WideSegs& ws, int wg, int waves, hipStream_t stream) {
  const size_t lds = (size_t)waves * T * NB4 * 64 * sizeof(float);
  hipLaunchKernelGGL((gemv_wide_kernel<NB4, T, WideChunk<NB4, T>::value>), dim3((unsigned)wg), dim3(64 * waves), lds,
                     stream, ws);
  return hipGetLastError();
}

// Tiles per wave: the most (up to kWideTMax, 4 above batch 8 where the
// accumulators crowd the registers) that still give the launch
// kWideMinWaves waves, else one.  More tiles per wave means fewer
// activation reads per tile; fewer waves leave CUs idle (the down projection,
// 320 tiles, takes two per wave).  Measured on the 27B-shaped layers.
template <int NB4>
hipError_t launch_wide(const GemvSegment* segs, int count, hipStream_t stream) {
  WideSegs ws{};
  int waves = 1;
  for (int T = NB4 <= 2 ? kWideTMax : std::min(kWideTMax, 4); T >= 1; T /= 2) {
    const int wg = wide_plan(segs, count, T, ws, waves);
    if (T > 1 && (int64_t)wg * waves < kWideMinWaves) continue;
    if constexpr (NB4 <= 2) {
      if (T == 8) return launch_wide_t<NB4, 8>(ws, wg, waves, stream);
    }
    if (T == 4) return launch_wide_t<NB4, 4>(ws, wg, waves, stream);
    if (T == 2) return launch_wide_t<NB4, 2>(ws, wg, waves, stream);
    return launch_wide_t<NB4, 1>(ws, wg, waves, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_multi(const GemvSegment* segs_in, int count, hipStream_t stream) {
  // one grouped launch when every segment takes the same path alone and the
  // group fits it, else each segment on its own exactly as a single call
  // would run it (a segment's result never depends on its companions, nor
  // on its place in the launch)
  //
  // The longest-K segments take the first workgroups: their workgroups carry
  // the most work (more K slices per tile), and dispatched last they would
  // set the launch's tail.  A 27B layer's four products in one launch at
  // batch 1: 20.2 -> 19.7 us, step 1.50 -> 1.48 ms; batch 8 34.7 -> 32.4 us.
  GemvSegment segs[kMaxSegs];
  if (count > kMaxSegs) {
    for (int c = 0; c < count; ++c) {
      const hipError_t e = launch_gemv_multi(segs_in + c, 1, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  std::copy(segs_in, segs_in + count, segs);
  std::stable_sort(segs, segs + count, [](const GemvSegment& a, const GemvSegment& b) {
    return a.K * a.planes > b.K * b.planes;
  });
  int n_staged = 0;
  for (int c = 0; c < count; ++c) n_staged += stageable(segs[c]) ? 1 : 0;
  if (count >= 1 && count <= kMaxSegs && n_staged == 0) {
    int bmax = 1;
    for (int c = 0; c < count; ++c) bmax = std::max(bmax, (int)segs[c].B);
    switch ((bmax + 3) / 4) {
      case 1:
        return launch_wide<1>(segs, count, stream);
      case 2:
        return launch_wide<2>(segs, count, stream);
      case 3:
        return launch_wide<3>(segs, count, stream);
      default:
        return launch_wide<4>(segs, count, stream);
    }
  }
  StagedSegs st{};
  bool staged = count <= kMaxSegs && n_staged == count;
  int bmax = 1, ch = 1, waves = 1, wg = 0;
  const int64_t planes = count > 0 ? segs[0].planes : 1;
  for (int c = 0; c < count && staged; ++c) {
    int ks = 0, sc = 0;
    staged_geometry(segs[c], ks, sc);
    bmax = std::max(bmax, (int)segs[c].B);
    ch = std::max(ch, sc);
    waves = std::max(waves, ks / (int)segs[c].parts);
    if (segs[c].planes != planes) staged = false;  // one plane count per grouped launch
  }
  // a slice of at most ch code groups spans at most ch activation groups with
  // one plane, ch / 2 + 1 with two
  const int stage_groups = planes == 1 ? ch : ch / 2 + 1;
  // Tiles per wave: 2 when every segment takes the short slices and the launch
  // has many tiles (one staged activation slice then serves two tiles; a 27B
  // layer's QKV + O + gate/up at batch 1: 16.4 -> 15.9 us), else 1.  A tile's
  // sum does not depend on it.
  int64_t all_tiles = 0;
  for (int c = 0; c < count; ++c) all_tiles += segs[c].N / 16;
  const int LT = ch == kStagedCH && all_tiles >= kTwoTileMin ? 2 : 1;
  const size_t lds = (size_t)waves * bmax * stage_groups * kStageBytes + (size_t)waves * LT * 64 * sizeof(float);
  if (staged && lds <= kStagedMaxLds) {
    for (int c = 0; c < count; ++c) {
      int ks = 0, sc = 0;
      staged_geometry(segs[c], ks, sc);
      const int parts = (int)segs[c].parts;
      const int64_t tiles = segs[c].N / 16, per_wg = waves / (ks / parts) * LT;
      st.s[c] = StagedSeg{segs[c].act, segs[c].codes, segs[c].scales, segs[c].y, segs[c].N, segs[c].K,
                          (int)segs[c].B, ks, wg, __builtin_ctz((unsigned)parts)};
      wg += (int)((tiles + per_wg - 1) / per_wg * parts);
    }
    st.count = count;
    st.bmax = bmax;
    st.stage_groups = stage_groups;
    const dim3 grid((unsigned)wg), block(64 * waves);
#define TB_STAGED(CH_, BMAX_, P_)                                                                \
  do {                                                                                           \
    if (LT == 2)                                                                                 \
      hipLaunchKernelGGL((gemv_staged_kernel<CH_, BMAX_, P_, 2>), grid, block, lds, stream, st); \
    else                                                                                         \
      hipLaunchKernelGGL((gemv_staged_kernel<CH_, BMAX_, P_, 1>), grid, block, lds, stream, st); \
  } while (0)
    // batch 1 only: kernels exist for 10 and 17 groups per wave
    if (planes == 1) {
      if (ch == kLongCH)
        TB_STAGED(kLongCH, 1, 1);
      else
        TB_STAGED(kStagedCH, 1, 1);
    } else {
      if (ch == kLongCH)
        TB_STAGED(kLongCH, 1, 2);
      else
        TB_STAGED(kStagedCH, 1, 2);
    }
#undef TB_STAGED
    return hipGetLastError();
  }
  if (count == 1) {
    // a stageable segment whose staging does not fit the LDS budget
    return launch_wide<1>(segs, 1, stream);
  }
  for (int c = 0; c < count; ++c) {
    const hipError_t e = launch_gemv_multi(segs + c, 1, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


}  // namespace tb
