// Shared device helpers for the libtb HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tb.h"

namespace tb {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) __bf16 bf16x16;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) uint32_t u32x8;

constexpr int kWave = 64;
constexpr int kBlock = 128;  // Hadamard block and scale group size

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// float -> fp16 bits (hardware conversion: round to nearest even, IEEE overflow to inf).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Value of lane (lane ^ 32): v_permlane32_swap exchanges the upper 32 lanes of
// its first operand with the lower 32 lanes of its second; with both operands v
// the pair comes back as (lower half broadcast, upper half broadcast).
__device__ __forceinline__ void swap_halves(float v, float& lower, float& upper) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lower = __uint_as_float(r[0]);
  upper = __uint_as_float(r[1]);
}

// Cross-lane exchange inside 16-lane rows by DPP / swizzle (no LDS traffic):
// returns v from lane (lane ^ MASK), MASK in {1, 2, 4, 8}.
template <int MASK>
__device__ __forceinline__ float xor_lane(float v) {
  int iv = __float_as_int(v);
  int r;
  if constexpr (MASK == 1) {
    r = __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (MASK == 2) {
    r = __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (MASK == 4) {
    r = __builtin_amdgcn_ds_swizzle(iv, 0x101F);  // bitmask mode: and 0x1f, xor 4
  } else {
    static_assert(MASK == 8, "mask");
    r = __builtin_amdgcn_update_dpp(0, iv, 0x128, 0xF, 0xF, false);  // row_ror:8
  }
  return __int_as_float(r);
}

// Keep the sources `a` and `b` of an instruction that produced `d` in vector
// registers until after it: the asm reads all three, so it cannot be placed
// before the instruction, and the sources stay live across it (their
// registers cannot be reused for `d`).  The asm exists only in the device
// pass: the host pass cannot parse the "v" constraint and would drop the
// kernel's launch stub.
template <typename D, typename A, typename B>
__device__ __forceinline__ void keep_sources_past(const D& d, const A& a, const B& b) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(d), "v"(a), "v"(b));
#else
  (void)d;
  (void)a;
  (void)b;
#endif
}

// Atomically OR `bits` into *flag once per wave (lanes with a nonzero `bits`).
__device__ __forceinline__ void wave_flag_or(int32_t* flag, uint32_t bits) {
  if (flag == nullptr) return;
  // reduce across the wave with a ballot per bit (only two flag bits exist)
  uint64_t b0 = __ballot((bits & 1u) != 0);
  uint64_t b1 = __ballot((bits & 2u) != 0);
  uint32_t all = (b0 ? 1u : 0u) | (b1 ? 2u : 0u);
  if (all != 0 && (threadIdx.x & (kWave - 1)) == 0) atomicOr(flag, (int32_t)all);
}

}  // namespace tb
