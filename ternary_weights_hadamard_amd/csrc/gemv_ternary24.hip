// Decode GEMV with 2:4 ternary weights (mhpq.cn/news/1159370 §1.2: two of
// every four kept, each kept element +-1 times the group scale):
//   y[b][n] = sum_g f16(scale[n][g]) * sum_q (+-x[b][4q + idx0] +- x[b][4q + idx1])
//
// gfx950's sparse matrix instruction v_smfmac_f32_16x16x64_bf16 takes a 16x64
// operand stored as 16x32 kept values plus a 2-bit position per kept value,
// two per quad, the first in the low bits: exactly the meta nibble of this
// format.  So the meta words go to the instruction untouched (the two 16-bit
// halves of one word are the two SMFMACs of a 128-group, picked by ABID), and
// the kept values are bf16 +-1 made from the sign field with one shift and
// one and-or per pair.
// Operand placement (from the instruction's layout): lane (i, q) supplies the
// kept values of row i for 16 consecutive sparse K and the dense x values of
// batch row i at two 8-wide K blocks; D[4q + r][i] returns in lane (i, q).
// The 64-wide windows are mapped to actual K so that lane q of SMFMAC h covers
// K 128g + 32q + 16h .. +15: one meta word and one sign field per lane and
// group.
//
// The planes are lane-major in blocks of four groups (a 16-row tile and four
// 128-groups together): lane 16q + i finds its meta words of the block's four
// groups in one 16-byte load, its four sign fields in one 8-byte load and the
// scales of its four output rows in the block's 128-byte scale record (an
// 8-byte load of one group's, moved across each quad of lanes).  With one
// meta, sign and scale load per group (the tile-major layout this replaced),
// a 17408 x 5120 launch issued three times as many load instructions and
// took 8.7-9.6 us against 7.9-8.2.
//
// Staged kernel (batch <= 4): a wave owns one 16-row tile and a slice of at
// most NBK blocks.  It issues its slice of x (16 bytes per lane per block and
// batch row) and then every weight load of the slice before any use, puts x
// in a private LDS area and reads it back in the operand layout.  The slices
// of a tile are the waves of one workgroup, added through LDS in a fixed
// order.  Direct kernel (larger batches, or slices too long to stage): the
// same loads in chunks of two blocks, x read from memory in the operand
// layout.
#include <algorithm>
#include <cstdlib>

#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

constexpr int kBlockGroups = 4;     // 128-groups per block of the stored format
constexpr int kBlockXBytes = 1024;  // bf16 x of one block and batch row
constexpr int kMaxSlices = 16;      // waves per workgroup
constexpr int kMaxResidentWaves = 6144;  // 24 per CU: more slices only add rounds
constexpr size_t kMaxLds = 160 * 1024;
// 16-row tiles per wave in a grouped launch.  Two (sharing the staged x)
// were slower on a 27B layer's four products: 37-38 us against 25-26 us
// per launch (88 registers, five waves per SIMD)
constexpr int kGroupedTiles = 1;

// the value of lane j of each quad of lanes, in all four (DPP quad_perm(j, j, j, j))
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v, int j) {
  switch (j) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, false);
  }
}

// Group j of a block for this lane: the 16-bit sign field (idx0 signs in bits
// 0-7, idx1 signs in bits 8-15) spread to bits 0-7 and 16-23, so that the
// signs of quad e sit at bits e and 16 + e like the sign bits of a bf16 pair:
// one byte permute (selector byte 0x0C gives zero).
__device__ __forceinline__ uint32_t sign_word(const u32x2& sw, int j) {
  const uint32_t w = sw[j >> 1];
  return __builtin_amdgcn_perm(w, w, (j & 1) ? 0x0C030C02u : 0x0C010C00u);
}

// bf16 +1 in both halves, in a VGPR: the kept-value build is then one
// shift and one and-or per dword (with the constant as an immediate the
// compiler split the and-or in two, as a VOP3 instruction here takes no
// literal and reads at most one SGPR).  The asm exists only in the device
// pass, like keep_sources_past: the host pass cannot parse the "v"
// constraint.
__device__ __forceinline__ uint32_t bf16_one_pair() {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t v;
  asm volatile("v_mov_b32 %0, 0x3f803f80" : "=v"(v));
  return v;
#else
  return 0x3F803F80u;
#endif
}

// SMFMAC h (0, 1) of a group for a lane: kept values of its quads 4h ..
// 4h + 3 from the sign word, dense operand bx (x chunks b0 + 2h and
// b0 + 2h + 8 of the group), meta word mw.
__device__ __forceinline__ f32x4 half_product(uint32_t mw, uint32_t sgw, int h, const u32x8& bx, f32x4 acc,
                                              uint32_t one) {
  u32x4 a;
#pragma unroll
  for (int d = 0; d < 4; ++d) a[d] = ((sgw << (15 - (4 * h + d))) & 0x80008000u) | one;
  if (h == 0)
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, bx),
                                                     acc, (int)mw, 0, 0);
  return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, bx),
                                                   acc, (int)mw, 0, 1);
}

// One group's two SMFMACs for a lane, x chunks b0 + 2h and b0 + 2h + 8 (16
// bytes each) of the group's 256 bytes from xload.
template <typename XLoad>
__device__ __forceinline__ f32x4 group_product(uint32_t mw, uint32_t sgw, int b0, XLoad xload, uint32_t one) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 lo = xload(b0 + 2 * h), hi = xload(b0 + 2 * h + 8);
    const u32x8 bx = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    acc = half_product(mw, sgw, h, bx, acc, one);
  }
  return acc;
}

// acc_y[r] += scale(row 4q + r, group j) * acc[r]; sc holds the lane's
// 8-byte piece of the block's scale record (group li % 4)
__device__ __forceinline__ void scale_add(f32x4& acc_y, const f32x4& acc, const u32x2& sc, int j) {
  const uint32_t s0 = quad_bcast(sc[0], j), s1 = quad_bcast(sc[1], j);
  const uint32_t sv[4] = {s0 & 0xFFFFu, s0 >> 16, s1 & 0xFFFFu, s1 >> 16};
#pragma unroll
  for (int r = 0; r < 4; ++r) acc_y[r] = __builtin_fmaf(f16_bits_to_f32(sv[r]), acc[r], acc_y[r]);
}

// the slices' partial sums added in wave order through LDS; wave 0 stores
__device__ __forceinline__ void reduce_store(f32x4 acc_y, float* red, int KS, int w, int lane, int li, int q, int B,
                                             float* y, int64_t N, int64_t nb) {
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

__host__ __device__ constexpr int stage24_bytes(int nbk, int bm) { return bm * nbk * kBlockXBytes; }

// One wave's slice of T consecutive tiles (nt <= T of them real): blocks
// [bb, bb + nblk) (1 <= nblk <= NBK) of each, tile u's first block at
// tile-block tb0 + u G4; at most four batch rows (BM = 1 for one).  It
// issues its slice of x (lane l: elements 8 l .. 8 l + 7 of each block,
// group l / 16, none past the last group) and then every weight load of the
// slice before any use, puts x in its own LDS area st_x and reads it back in
// the operand layout, once for all T tiles.  acc_y[u] receives the lane's
// partial sums of y[li][16 tile_u + 4q + r].
template <int NBK, int BM, int T>
__device__ __forceinline__ void slice_sum(const uint16_t* __restrict__ x, int B, int64_t K, int G, int G4,
                                          const uint32_t* __restrict__ meta, const uint32_t* __restrict__ signs,
                                          const uint16_t* __restrict__ scales, int64_t tb0, int nt, int bb, int nblk,
                                          unsigned char* st_x, int lane, f32x4 (&acc_y)[T]) {
  const int li = lane & 15, q = lane >> 4;
  const int ng = min(4 * nblk, G - 4 * bb);  // groups of the slice
  u32x4 x_st[BM][NBK];
#pragma unroll
  for (int b = 0; b < BM; ++b)
#pragma unroll
    for (int t = 0; t < NBK; ++t)
      if (t < nblk && b < B && 4 * t + (lane >> 4) < ng)
        x_st[b][t] = *reinterpret_cast<const u32x4*>(x + (int64_t)b * K + 512 * (bb + t) + 8 * lane);
  u32x4 mw[T][NBK];
  u32x2 sw[T][NBK], sc[T][NBK];
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int t = 0; t < NBK; ++t) {
      if (u < nt && t < nblk) {
        const int64_t tbk = tb0 + (int64_t)u * G4 + t;
        mw[u][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(meta) + tbk * 64 + lane);
        sw[u][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(signs) + tbk * 64 + lane);
        sc[u][t] = *reinterpret_cast<const u32x2*>(scales + tbk * 64 + 4 * (4 * q + (li & 3)));
        // a group past K (padding of the last block) takes scale 0 whatever
        // the stored planes hold there
        if (4 * t + (li & 3) >= ng) sc[u][t] = u32x2{0u, 0u};
      }
    }
  // groups past K stage zeros, so with scale 0 they add exactly nothing
#pragma unroll
  for (int b = 0; b < BM; ++b)
#pragma unroll
    for (int t = 0; t < NBK; ++t)
      if (t < nblk && b < B)
        *reinterpret_cast<u32x4*>(st_x + (b * NBK + t) * kBlockXBytes + 16 * lane) =
            4 * t + (lane >> 4) < ng ? x_st[b][t] : u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // Lanes of batch rows >= B read row B - 1 (their results are never
  // stored).  Blocks past the slice are a wave-uniform branch; every group
  // of a block runs (straight-line code: a branch per group cost 20 % on a
  // 27B layer's grouped launch).
  const int b0 = 4 * (q >> 1) + (q & 1);
  const unsigned char* xrow = st_x + (BM == 1 ? 0 : (size_t)min(li, B - 1) * NBK * kBlockXBytes);
  const uint32_t one = bf16_one_pair();
#pragma unroll
  for (int u = 0; u < T; ++u) acc_y[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NBK; ++t) {
    if (t < nblk) {
#pragma unroll
      for (int j = 0; j < kBlockGroups; ++j) {
        const unsigned char* xg = xrow + t * kBlockXBytes + j * 256;
        f32x4 acc[T];
#pragma unroll
        for (int u = 0; u < T; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(xg + 16 * (b0 + 2 * h));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(xg + 16 * (b0 + 2 * h + 8));
          const u32x8 bx = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int u = 0; u < T; ++u)
            if (u < nt) acc[u] = half_product(mw[u][t][j], sign_word(sw[u][t], j), h, bx, acc[u], one);
        }
#pragma unroll
        for (int u = 0; u < T; ++u)
          if (u < nt) scale_add(acc_y[u], acc[u], sc[u][t], j);
      }
    }
  }
}

// Block size 64 * KS: wave w takes blocks [w NBK, w NBK + NBK) of tile
// blockIdx.x (the launch guarantees (KS - 1) NBK < G4).
template <int NBK, int BM>
__global__ void __launch_bounds__(1024) gemv24_staged_kernel(const uint16_t* __restrict__ x, int B,
                                                             const uint32_t* __restrict__ meta,
                                                             const uint32_t* __restrict__ signs,
                                                             const uint16_t* __restrict__ scales, int64_t N,
                                                             int64_t K, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int KS = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nb = blockIdx.x;
  const int G = (int)((uint64_t)K >> 7);
  const int G4 = (G + kBlockGroups - 1) / kBlockGroups;
  const int bb = w * NBK;
  const int nblk = min(NBK, G4 - bb);
  unsigned char* st_x = smem + (size_t)w * stage24_bytes(NBK, BM);
  float* red = reinterpret_cast<float*>(smem + (size_t)KS * stage24_bytes(NBK, BM));
  f32x4 acc_y[1];
  slice_sum<NBK, BM, 1>(x, B, K, G, G4, meta, signs, scales, nb * G4 + bb, 1, bb, nblk, st_x, lane, acc_y);
  reduce_store(acc_y[0], red, KS, w, lane, lane & 15, lane >> 4, B, y, N, nb);
}

// Several products in one launch.  Segment c owns workgroups [wg_begin,
// next segment's wg_begin); each of its workgroups takes tpw groups of T
// consecutive tiles, each group wpt waves of nbk blocks (tpw wpt <= KS;
// waves past them only join the barrier).
struct G24Seg {
  const uint16_t* x;
  const uint32_t* meta;
  const uint32_t* signs;
  const uint16_t* scales;
  float* y;
  int64_t N, K;
  int B, wg_begin, tpw, wpt, nbk, reserved;
};

struct G24Segs {
  G24Seg s[TB_MAX_SEGMENTS];
  int count;
};

template <int NBK, int BM, int T>
__global__ void __launch_bounds__(1024) gemv24_grouped_kernel(G24Segs segs) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int KS = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, q = lane >> 4;
  int seg = 0;
#pragma unroll
  for (int t = 1; t < TB_MAX_SEGMENTS; ++t)
    seg += (t < segs.count && (int)blockIdx.x >= segs.s[t].wg_begin) ? 1 : 0;
  const G24Seg& sg = segs.s[seg];
  const int u = w / sg.wpt, v = w - u * sg.wpt;  // tile group of the workgroup, slice of the tiles
  const int64_t tiles = sg.N / 16;
  const int64_t tile0 = ((int64_t)((int)blockIdx.x - sg.wg_begin) * sg.tpw + u) * T;
  const bool active = u < sg.tpw && tile0 < tiles;
  const int nt = (int)min((int64_t)T, tiles - tile0);
  unsigned char* st_x = smem + (size_t)w * stage24_bytes(NBK, BM);
  float* red = reinterpret_cast<float*>(smem + (size_t)KS * stage24_bytes(NBK, BM));
  f32x4 acc_y[T];
  if (active) {
    const int G = (int)((uint64_t)sg.K >> 7);
    const int G4 = (G + kBlockGroups - 1) / kBlockGroups;
    const int bb = v * sg.nbk;
    slice_sum<NBK, BM, T>(sg.x, sg.B, sg.K, G, G4, sg.meta, sg.signs, sg.scales, tile0 * G4 + bb, nt, bb,
                          min(sg.nbk, G4 - bb), st_x, lane, acc_y);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((w * T + t) * 4 + r) * 64 + lane] = acc_y[t][r];
  }
  __syncthreads();
  if (active && v == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        for (int o = 1; o < sg.wpt; ++o) acc_y[t][r] += red[(((w + o) * T + t) * 4 + r) * 64 + lane];
      if (t < nt && li < sg.B)
        *reinterpret_cast<f32x4*>(sg.y + (int64_t)li * sg.N + 16 * (tile0 + t) + 4 * q) = acc_y[t];
    }
  }
}

// Direct kernel, any B <= 16: wave w takes blocks [w spb, min(G4, w spb +
// spb)) of tile blockIdx.x, two blocks at a time, x straight from memory.
__global__ void __launch_bounds__(1024) gemv24_direct_kernel(const uint16_t* __restrict__ x, int B,
                                                             const uint32_t* __restrict__ meta,
                                                             const uint32_t* __restrict__ signs,
                                                             const uint16_t* __restrict__ scales, int64_t N,
                                                             int64_t K, float* __restrict__ y, int spb) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int kChunk = 2;
  const int KS = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, q = lane >> 4;
  const int64_t nb = blockIdx.x;
  const int G = (int)((uint64_t)K >> 7);
  const int G4 = (G + kBlockGroups - 1) / kBlockGroups;
  const int bb = w * spb, be = min(G4, bb + spb);
  float* red = reinterpret_cast<float*>(smem);
  const int b0 = 4 * (q >> 1) + (q & 1);
  const uint16_t* xrow = x + (int64_t)min(li, B - 1) * K;
  const uint32_t one = bf16_one_pair();
  f32x4 acc_y = {0.f, 0.f, 0.f, 0.f};
  for (int c = bb; c < be; c += kChunk) {
    u32x4 mw[kChunk];
    u32x2 sw[kChunk], sc[kChunk];
#pragma unroll
    for (int t = 0; t < kChunk; ++t) {
      const int64_t tbk = nb * G4 + min(c + t, be - 1);
      mw[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(meta) + tbk * 64 + lane);
      sw[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(signs) + tbk * 64 + lane);
      sc[t] = *reinterpret_cast<const u32x2*>(scales + tbk * 64 + 4 * (4 * q + (li & 3)));
    }
#pragma unroll
    for (int t = 0; t < kChunk; ++t) {
#pragma unroll
      for (int j = 0; j < kBlockGroups; ++j) {
        const int g = 4 * (c + t) + j;
        if (c + t >= be || g >= G) break;
        const uint16_t* xg = xrow + (int64_t)128 * g;
        const f32x4 acc = group_product(mw[t][j], sign_word(sw[t], j), b0, [&](int cc) {
          return *reinterpret_cast<const u32x4*>(xg + 8 * cc);
        }, one);
        scale_add(acc_y, acc, sc[t], j);
      }
    }
  }
  reduce_store(acc_y, red, KS, w, lane, li, q, B, y, N, nb);
}

template <int NBK>
void launch_staged(int bm, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const uint16_t* x, int B,
                   const uint32_t* meta, const uint32_t* signs, const uint16_t* scales, int64_t N, int64_t K,
                   float* y) {
  if (bm == 1)
    hipLaunchKernelGGL((gemv24_staged_kernel<NBK, 1>), grid, block, lds, stream, x, B, meta, signs, scales, N, K, y);
  else
    hipLaunchKernelGGL((gemv24_staged_kernel<NBK, 4>), grid, block, lds, stream, x, B, meta, signs, scales, N, K, y);
}

template <int NBK, int T>
void launch_grouped(int bm, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const G24Segs& segs) {
  if (bm == 1)
    hipLaunchKernelGGL((gemv24_grouped_kernel<NBK, 1, T>), grid, block, lds, stream, segs);
  else
    hipLaunchKernelGGL((gemv24_grouped_kernel<NBK, 4, T>), grid, block, lds, stream, segs);
}

template <int T>
void launch_grouped_t(int nbk, int bm, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const G24Segs& segs) {
  switch (nbk) {
    case 1: launch_grouped<1, T>(bm, grid, block, lds, stream, segs); break;
    case 2: launch_grouped<2, T>(bm, grid, block, lds, stream, segs); break;
    case 3: launch_grouped<3, T>(bm, grid, block, lds, stream, segs); break;
    default: launch_grouped<4, T>(bm, grid, block, lds, stream, segs); break;
  }
}

// LDS of a grouped launch: each wave's x area and its T tiles' partial sums
size_t grouped_lds(int ks, int nbk, int bm, int T) {
  return (size_t)ks * (stage24_bytes(nbk, bm) + (size_t)T * 4 * 64 * sizeof(float));
}

// Geometry of a grouped launch: waves per workgroup ks and, per segment,
// blocks per wave, waves per tile and tiles per workgroup.  Over ks = 1..16
// each segment takes the blocks per wave (1..4) that leave the fewest idle
// waves in its workgroups (ties: the one nearest 2, the single-launch
// optimum), weighted by its work; the launch takes the largest ks that keeps
// at least 90 % of the work on busy waves (a 27B layer: 16 waves, 24.9 us,
// against 25.7-26.5 us with the 12 that leave none idle).
struct G24Geometry {
  int ks = 0, nbk_max = 0, tiles_per_wave = 1;
  int nbk[TB_MAX_SEGMENTS], wpt[TB_MAX_SEGMENTS], tpw[TB_MAX_SEGMENTS];
};

G24Geometry grouped_geometry(const tb_gemv24_segment* segs, int count, int bm, int T) {
  G24Geometry best;
  double best_util = -1.0;
  for (int ks = 1; ks <= kMaxSlices; ++ks) {
    G24Geometry g;
    g.ks = ks;
    double busy = 0.0, total = 0.0;
    bool ok = true;
    for (int c = 0; c < count && ok; ++c) {
      const int64_t G4 = (segs[c].K / kBlock + kBlockGroups - 1) / kBlockGroups;
      int pick = 0;
      double pick_u = -1.0;
      for (int nbk = 1; nbk <= 4; ++nbk) {
        const int64_t wpt = (G4 + nbk - 1) / nbk;
        if (wpt > ks) continue;
        const double u = (double)(ks / wpt * wpt) / ks;
        if (u > pick_u + 1e-9 || (u > pick_u - 1e-9 && std::abs(nbk - 2) < std::abs(pick - 2))) {
          pick = nbk;
          pick_u = u;
        }
      }
      if (pick == 0) {
        ok = false;
        break;
      }
      g.nbk[c] = pick;
      g.wpt[c] = (int)((G4 + pick - 1) / pick);
      g.tpw[c] = ks / g.wpt[c];
      g.nbk_max = std::max(g.nbk_max, pick);
      const double work = (double)(segs[c].N / 16) * (double)G4;
      busy += work * pick_u;
      total += work;
    }
    if (!ok) continue;
    if (grouped_lds(ks, g.nbk_max, bm, T) > kMaxLds) continue;
    g.tiles_per_wave = T;
    const double util = busy / total;
    const bool good = util >= 0.9, best_good = best_util >= 0.9;
    if (best.ks == 0 || good || (!best_good && util > best_util)) {
      best = g;
      best_util = util;
    }
  }
  return best;
}

}  // namespace

hipError_t launch_gemv24_multi(const tb_gemv24_segment* segs, int count, hipStream_t stream) {
  // (segments stay in the caller's order: longest K first measured the same
  // on a 27B layer, 25.4-25.9 against 25.1-25.5 us)
  // one product: its own launch geometry (many small workgroups; the grouped
  // geometry's large ones measured 5120 x 5120 8.0 against 4.4 us, 17408 x
  // 5120 11.7 against 7.9 us), and the single call's result bit for bit
  if (count == 1)
    return launch_gemv_ternary24(segs[0].x, segs[0].B, segs[0].meta, segs[0].signs, segs[0].scales, segs[0].N,
                                 segs[0].K, segs[0].y, stream);
  bool staged = count <= TB_MAX_SEGMENTS;
  int bm = 1;
  for (int c = 0; c < count; ++c) {
    staged = staged && segs[c].B <= 4;
    if (segs[c].B > 1) bm = 4;
  }
  const G24Geometry g = staged ? grouped_geometry(segs, count, bm, kGroupedTiles) : G24Geometry{};
  if (g.ks == 0) {
    // batches past 4 or rows too long to stage: one launch per product
    for (int c = 0; c < count; ++c) {
      const tb_gemv24_segment& a = segs[c];
      const hipError_t e = launch_gemv_ternary24(a.x, a.B, a.meta, a.signs, a.scales, a.N, a.K, a.y, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  G24Segs gs{};
  int64_t wgs = 0;
  for (int c = 0; c < count; ++c) {
    const tb_gemv24_segment& a = segs[c];
    const int64_t groups = (a.N / 16 + g.tiles_per_wave - 1) / g.tiles_per_wave;
    gs.s[c] = G24Seg{a.x, a.meta, a.signs, a.scales, a.y, a.N, a.K, (int)a.B, (int)wgs, g.tpw[c], g.wpt[c],
                     g.nbk[c], 0};
    wgs += (groups + g.tpw[c] - 1) / g.tpw[c];
  }
  gs.count = count;
  if (wgs == 0) return hipSuccess;
  if (wgs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const size_t lds = grouped_lds(g.ks, g.nbk_max, bm, g.tiles_per_wave);
  const dim3 grid((unsigned)wgs), block((unsigned)(64 * g.ks));
  static_assert(kGroupedTiles == 1, "one tile per wave is the instantiated grouped kernel");
  launch_grouped_t<1>(g.nbk_max, bm, grid, block, lds, stream, gs);
  return hipGetLastError();
}

hipError_t launch_gemv_ternary24(const uint16_t* x, int64_t B, const uint32_t* meta, const uint32_t* signs,
                                 const uint16_t* scales, int64_t N, int64_t K, float* y, hipStream_t stream) {
  const int64_t G = K / kBlock;
  const int64_t G4 = (G + kBlockGroups - 1) / kBlockGroups;
  const int64_t tiles = N / 16;
  const size_t red_bytes = 4 * 64 * sizeof(float);  // per wave
  if (B <= 4) {
    // Staged: the fewest blocks per wave (NBK <= 4, at most 16 slices) that
    // keep every wave of the launch resident at once (about 24 per CU), else
    // the largest that fits.  Per launch, batch 1: 17408 x 5120 takes 2 blocks
    // per wave (1: 8.9 us, 2: 7.9, 3: 8.6); 5120 x 5120 takes 1 (4.6 against
    // 5.0 with 2); 5120 x 17408 takes 3 (10.0 us; 4: 10.1).
    const int bm = B == 1 ? 1 : 4;
    int pick = 0;
    for (int nbk = 1; nbk <= 4; ++nbk) {
      const int64_t ks = (G4 + nbk - 1) / nbk;
      const size_t lds = (size_t)ks * (stage24_bytes(nbk, bm) + red_bytes);
      if (ks > kMaxSlices || lds > kMaxLds) continue;
      pick = nbk;
      if (tiles * ks <= kMaxResidentWaves) break;
    }
    if (pick > 0) {
      const int64_t ks = (G4 + pick - 1) / pick;
      const size_t lds = (size_t)ks * (stage24_bytes(pick, bm) + red_bytes);
      const dim3 grid((unsigned)tiles), block((unsigned)(64 * ks));
      switch (pick) {
        case 1: launch_staged<1>(bm, grid, block, lds, stream, x, (int)B, meta, signs, scales, N, K, y); break;
        case 2: launch_staged<2>(bm, grid, block, lds, stream, x, (int)B, meta, signs, scales, N, K, y); break;
        case 3: launch_staged<3>(bm, grid, block, lds, stream, x, (int)B, meta, signs, scales, N, K, y); break;
        default: launch_staged<4>(bm, grid, block, lds, stream, x, (int)B, meta, signs, scales, N, K, y); break;
      }
      return hipGetLastError();
    }
  }
  const int64_t ks = std::min<int64_t>(kMaxSlices, G4);
  const int64_t spb = (G4 + ks - 1) / ks;
  const int64_t used = (G4 + spb - 1) / spb;  // every wave keeps at least one block
  const dim3 grid((unsigned)tiles), block((unsigned)(64 * used));
  hipLaunchKernelGGL(gemv24_direct_kernel, grid, block, (size_t)used * red_bytes, stream, x, (int)B, meta, signs,
                     scales, N, K, y, (int)spb);
  return hipGetLastError();
}

}  // namespace tb
