// Measurement probes (include/tb_probe.h): the achievable HBM read bandwidth
// and bf16 matrix-instruction rate of the device, measured with the simplest
// kernels that reach them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tb_probe.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

constexpr int kWaves = 4;
constexpr int kLoads = 4;  // 16-byte loads per lane in flight: 4 KB per wave step

__global__ void __launch_bounds__(64 * kWaves) stream_read_kernel(const uint8_t* __restrict__ src, size_t nbytes,
                                                                   uint32_t* __restrict__ sink) {
  const size_t wave = (size_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const size_t nwaves = (size_t)gridDim.x * kWaves;
  const int lane = threadIdx.x & 63;
  constexpr size_t kStep = 64 * 16 * kLoads;
  uint32_t fold = 0;
  for (size_t base = wave * kStep; base + kStep <= nbytes; base += nwaves * kStep) {
    u32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + base + (size_t)u * 1024 + lane * 16));
#pragma unroll
    for (int u = 0; u < kLoads; ++u) fold ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (fold == 0x9E3779B9u) sink[wave * 64 + lane] = fold;
}

__global__ void __launch_bounds__(64 * kWaves) mfma_bf16_kernel(float* __restrict__ sink, int iters) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((t + e) & 7);
    b[e] = (__bf16)(float)((t * 3 + e) & 7);
  }
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
  }
  sink[(size_t)blockIdx.x * 64 * kWaves + t] = (c0[0] + c1[1]) + (c2[2] + c3[3]);
}

}  // namespace

extern "C" {

int tbp_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, void* stream) {
  if (!src || !sink || grid <= 0 || (bytes & 4095) != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(64 * kWaves), 0, (hipStream_t)stream,
                     static_cast<const uint8_t*>(src), bytes, sink);
  return (int)hipGetLastError();
}

int tbp_mfma_bf16(float* sink, int iters, int grid, void* stream) {
  if (!sink || grid <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3((unsigned)grid), dim3(64 * kWaves), 0, (hipStream_t)stream, sink, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
