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

#include "tb_common.h"
#include "tb_launch.h"

namespace tb {

namespace {

constexpr int kBlockGroups = 4;     // 128-groups per block of the stored format
constexpr int kBlockXBytes = 1024;  // bf16 x of one block and batch row
constexpr int kMaxSlices = 16;      // waves per workgroup
constexpr int kMaxResidentWaves = 6144;  // 24 per CU: more slices only add rounds
constexpr size_t kMaxLds = 160 * 1024;

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
// signs of quad e sit at bits e and 16 + e like the sign bits of a bf16 pair.
__device__ __forceinline__ uint32_t sign_word(const u32x2& sw, int j) {
  const uint32_t f = sw[j >> 1] >> (16 * (j & 1));
  return (f & 0xFFu) | ((f & 0xFF00u) << 8);
}

// One group's two SMFMACs for a lane: kept values of quads 4h .. 4h + 3 from
// the sign word, x chunks b0 + 2h and b0 + 2h + 8 (16 bytes each) of the
// group's 256 bytes at xg.
template <typename XLoad>
__device__ __forceinline__ f32x4 group_product(uint32_t mw, uint32_t sgw, int b0, XLoad xload) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 a;
#pragma unroll
    for (int d = 0; d < 4; ++d) a[d] = ((sgw << (15 - (4 * h + d))) & 0x80008000u) | 0x3F803F80u;
    const u32x4 lo = xload(b0 + 2 * h), hi = xload(b0 + 2 * h + 8);
    const u32x8 bx = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if (h == 0)
      acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, bx),
                                                      acc, (int)mw, 0, 0);
    else
      acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, bx),
                                                      acc, (int)mw, 0, 1);
  }
  return acc;
}

// acc_y[r] += scale(row 4q + r, group j) * acc[r] when `valid`; sc holds the
// lane's 8-byte piece of the block's scale record (group li % 4).
__device__ __forceinline__ void scale_add(f32x4& acc_y, const f32x4& acc, const u32x2& sc, int j, bool valid) {
  const uint32_t s0 = quad_bcast(sc[0], j), s1 = quad_bcast(sc[1], j);
  const uint32_t sv[4] = {s0 & 0xFFFFu, s0 >> 16, s1 & 0xFFFFu, s1 >> 16};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float v = __builtin_fmaf(f16_bits_to_f32(sv[r]), acc[r], acc_y[r]);
    acc_y[r] = valid ? v : acc_y[r];
  }
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

// Block size 64 * KS: wave w takes blocks [w NBK, w NBK + NBK) of tile
// blockIdx.x (the launch guarantees (KS - 1) NBK < G4).  BM = 1 for one
// batch row, 4 for up to four.
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
  const int li = lane & 15, q = lane >> 4;
  const int64_t nb = blockIdx.x;
  const int G = (int)((uint64_t)K >> 7);
  const int G4 = (G + kBlockGroups - 1) / kBlockGroups;
  const int bb = w * NBK;
  const int nblk = min(NBK, G4 - bb);          // 1 .. NBK blocks
  const int ng = min(4 * nblk, G - 4 * bb);    // groups of the slice
  unsigned char* st_x = smem + (size_t)w * stage24_bytes(NBK, BM);
  float* red = reinterpret_cast<float*>(smem + (size_t)KS * stage24_bytes(NBK, BM));

  // 1. the slice of x: lane l takes elements 8 l .. 8 l + 7 of each block
  //    (group l / 16 of the block), none past the slice's last group
  u32x4 x_st[BM][NBK];
#pragma unroll
  for (int b = 0; b < BM; ++b)
#pragma unroll
    for (int t = 0; t < NBK; ++t)
      if (b < B && 4 * t + (lane >> 4) < ng)
        x_st[b][t] = *reinterpret_cast<const u32x4*>(x + (int64_t)b * K + 512 * (bb + t) + 8 * lane);
  // 2. every weight load of the slice (slots past it repeat its last block)
  const int64_t tb0 = nb * G4 + bb;
  u32x4 mw[NBK];
  u32x2 sw[NBK], sc[NBK];
#pragma unroll
  for (int t = 0; t < NBK; ++t) {
    const int64_t tbk = tb0 + min(t, nblk - 1);
    mw[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(meta) + tbk * 64 + lane);
    sw[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(signs) + tbk * 64 + lane);
    sc[t] = *reinterpret_cast<const u32x2*>(scales + tbk * 64 + 4 * (4 * q + (li & 3)));
  }
  // 3. x into this wave's LDS area (read back by the same wave only)
#pragma unroll
  for (int b = 0; b < BM; ++b)
#pragma unroll
    for (int t = 0; t < NBK; ++t)
      if (b < B && 4 * t + (lane >> 4) < ng)
        *reinterpret_cast<u32x4*>(st_x + (b * NBK + t) * kBlockXBytes + 16 * lane) = x_st[b][t];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // 4. the products.  Lanes of batch rows >= B read row B - 1 (their results
  //    are never stored); groups past the slice are computed on whatever the
  //    LDS holds and dropped by the select in scale_add.
  const int b0 = 4 * (q >> 1) + (q & 1);
  const unsigned char* xrow = st_x + (BM == 1 ? 0 : (size_t)min(li, B - 1) * NBK * kBlockXBytes);
  f32x4 acc_y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NBK; ++t) {
    const int tt = min(t, nblk - 1);
#pragma unroll
    for (int j = 0; j < kBlockGroups; ++j) {
      const unsigned char* xg = xrow + tt * kBlockXBytes + j * 256;
      const f32x4 acc = group_product(mw[t][j], sign_word(sw[t], j), b0, [&](int c) {
        return *reinterpret_cast<const u32x4*>(xg + 16 * c);
      });
      scale_add(acc_y, acc, sc[t], j, 4 * t + j < ng);
    }
  }
  reduce_store(acc_y, red, KS, w, lane, li, q, B, y, N, nb);
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
        const bool valid = c + t < be && g < G;
        const uint16_t* xg = xrow + (int64_t)128 * min(g, G - 1);
        const f32x4 acc = group_product(mw[t][j], sign_word(sw[t], j), b0, [&](int cc) {
          return *reinterpret_cast<const u32x4*>(xg + 8 * cc);
        });
        scale_add(acc_y, acc, sc[t], j, valid);
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

}  // namespace

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
