// Internal launchers, one per kernel family.  Arguments are already validated
// by the C ABI layer (tb_api.hip); each returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tb.h"

namespace tb {

hipError_t launch_fwht128(const void* x, int x_dtype, void* y, int y_dtype, int64_t rows, int64_t K,
                          hipStream_t stream);
hipError_t launch_fwht128_multi(const tb_fwht_segment* segs, int count, hipStream_t stream);
hipError_t launch_quantize128(const float* W, int64_t N, int64_t K, int fmt, uint32_t* codes, uint32_t* meta,
                              uint16_t* scales, int32_t* err_flag, hipStream_t stream);
hipError_t launch_act8_prep(const uint16_t* x, int64_t rows, int64_t K, uint8_t* act, hipStream_t stream);
typedef tb_gemv_segment GemvSegment;
// segments' `planes` must be 1 or 2 and `parts` 1, 2, 4 or 8 (the API layer
// normalises both)
hipError_t launch_gemv_multi(const GemvSegment* segs, int count, hipStream_t stream);
hipError_t launch_gemv_ternary24(const uint16_t* x, int64_t B, const uint32_t* meta, const uint32_t* signs,
                                 const uint16_t* scales, int64_t N, int64_t K, float* y, hipStream_t stream);
// segments with B == 0 removed by the API layer
hipError_t launch_gemv24_multi(const tb_gemv24_segment* segs, int count, hipStream_t stream);
hipError_t launch_gemm_ternary(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                               int64_t N, int64_t K, void* y, int y_dtype, hipStream_t stream);
// at most this many activation rows take the mid-batch kernel (gemm_skinny.hip)
constexpr int kSkinnyMaxRows = 16;
// waves per workgroup of the mid-batch kernel for this shape
int gemm_skinny_waves(int64_t N, int64_t K);
// 1 <= M <= kSkinnyMaxRows; one pass, no workspace
hipError_t launch_gemm_skinny(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                              int64_t N, int64_t K, void* y, int y_dtype, hipStream_t stream);
// one launch of the mid-batch kernel over several products, every M <= kSkinnyMaxRows
hipError_t launch_gemm_skinny_multi(const tb_gemm_segment* segs, int count, hipStream_t stream);
// K splits the split-K GEMM uses for this shape (1: none)
int gemm_splitk_parts(int64_t M, int64_t N, int64_t K);
// split K when the workspace allows (else one pass); `rotate` rotates the
// result back along N (y = R_N y') before it is written
hipError_t launch_gemm_ternary_splitk(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                      int64_t N, int64_t K, void* y, int y_dtype, float* workspace,
                                      size_t workspace_bytes, bool rotate, hipStream_t stream);

}  // namespace tb
