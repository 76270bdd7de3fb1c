// C ABI of libtb: host-side argument validation, then one launch on the
// caller's stream.  Validation makes no HIP call, so every error path can be
// exercised without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tb.h"
#include "tb_launch.h"

namespace {

constexpr int64_t kGroup = 128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dims_ok(int64_t N, int64_t K) { return N > 0 && K > 0 && N % kGroup == 0 && K % kGroup == 0; }
bool dtype_ok(int d) { return d == TB_F32 || d == TB_BF16; }
size_t dtype_bytes(int d) { return d == TB_F32 ? 4 : 2; }
// bytes of the act8 operand of `elems` activations (4 per element + 1/8 of scales)
size_t act8_bytes(size_t elems) { return elems * 4 + elems / 8; }

// [a, a + na) and [b, b + nb) intersect (byte ranges)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return na && nb && pa < pb + nb && pb < pa + na;
}

tb_status launched(hipError_t e) { return e == hipSuccess ? TB_OK : TB_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// byte sizes of one FWHT segment's input and output
size_t fwht_in_bytes(int64_t rows, int64_t K, int x_dtype) { return (size_t)rows * (size_t)K * dtype_bytes(x_dtype); }
size_t fwht_out_bytes(int64_t rows, int64_t K, int y_dtype) {
  const size_t n = (size_t)rows * (size_t)K;
  return y_dtype == TB_ACT8 ? act8_bytes(n) : n * dtype_bytes(y_dtype);
}

tb_status check_fwht(const void* x, int x_dtype, const void* y, int y_dtype, int64_t rows, int64_t K) {
  if (!dtype_ok(x_dtype) || !(dtype_ok(y_dtype) || y_dtype == TB_ACT8)) return TB_ERR_DTYPE;
  if (rows < 0 || K <= 0 || K % kGroup) return TB_ERR_SHAPE;
  if (rows == 0) return TB_OK;
  if (!x || !y) return TB_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return TB_ERR_ALIGN;
  if (x == y && x_dtype != y_dtype) return TB_ERR_ALIAS;
  if (x != y && overlap(x, fwht_in_bytes(rows, K, x_dtype), y, fwht_out_bytes(rows, K, y_dtype))) return TB_ERR_ALIAS;
  return TB_OK;
}

// code planes of a GEMV segment (0 is read as 1), or 0 when invalid
int64_t gemv_planes(const tb_gemv_segment& g) { return g.planes == 0 ? 1 : (g.planes == 1 || g.planes == 2) ? g.planes : 0; }

// K parts of a GEMV segment (0 is read as 1), or 0 when invalid
int64_t gemv_parts(const tb_gemv_segment& g) {
  return g.parts == 0 || g.parts == 1 ? 1 : (g.parts == 2 || g.parts == 4 || g.parts == 8) ? g.parts : 0;
}

// bytes of a GEMV segment's output: its parts of [B][N] fp32
size_t gemv_y_bytes(const tb_gemv_segment& g) { return (size_t)gemv_parts(g) * (size_t)g.B * (size_t)g.N * 4; }

// bytes of a GEMV segment's codes and scales (all planes)
size_t gemv_code_bytes(const tb_gemv_segment& g) { return (size_t)gemv_planes(g) * (size_t)g.N * (size_t)g.K / 4; }
size_t gemv_scale_bytes(const tb_gemv_segment& g) { return (size_t)gemv_planes(g) * (size_t)g.N * (size_t)g.K / 64; }

tb_status check_gemv(const tb_gemv_segment& g) {
  if (gemv_planes(g) == 0) return TB_ERR_FORMAT;
  if (!dims_ok(g.N, g.K) || g.B < 0 || g.B > TB_GEMV_MAX_BATCH || gemv_parts(g) == 0) return TB_ERR_SHAPE;
  if (gemv_parts(g) > 1) {
    if (g.K / kGroup * gemv_planes(g) < gemv_parts(g)) return TB_ERR_SHAPE;  // every part at least one group
  }
  if (g.B == 0) return TB_OK;
  if (!g.act || !g.codes || !g.scales || !g.y) return TB_ERR_NULL;
  if (!aligned16(g.act) || !aligned16(g.codes) || !aligned16(g.scales) || !aligned16(g.y)) return TB_ERR_ALIGN;
  const size_t yb = gemv_y_bytes(g);
  if (overlap(g.y, yb, g.act, act8_bytes((size_t)g.B * g.K)) || overlap(g.y, yb, g.codes, gemv_code_bytes(g)) ||
      overlap(g.y, yb, g.scales, gemv_scale_bytes(g)))
    return TB_ERR_ALIAS;
  return TB_OK;
}

// The checks of a GEMV call with bf16 activations x [B][K] other than those of
// its act8 workspace (g.act is not looked at).
tb_status check_gemv_bf16(const void* x, const tb_gemv_segment& g) {
  if (gemv_planes(g) == 0) return TB_ERR_FORMAT;
  if (!dims_ok(g.N, g.K) || g.B < 0 || g.B > TB_GEMV_MAX_BATCH) return TB_ERR_SHAPE;
  if (g.B == 0) return TB_OK;
  if (!x || !g.codes || !g.scales || !g.y) return TB_ERR_NULL;
  if (!aligned16(x) || !aligned16(g.codes) || !aligned16(g.scales) || !aligned16(g.y)) return TB_ERR_ALIGN;
  const size_t yb = (size_t)g.B * (size_t)g.N * 4;
  if (overlap(g.y, yb, x, (size_t)g.B * (size_t)g.K * 2) || overlap(g.y, yb, g.codes, gemv_code_bytes(g)) ||
      overlap(g.y, yb, g.scales, gemv_scale_bytes(g)))
    return TB_ERR_ALIAS;
  return TB_OK;
}

// Encode bf16 x' as the act8 operand into g.act, then the product: two
// launches on the stream.
tb_status encode_and_multiply(const void* x, const tb_gemv_segment& g, hipStream_t stream) {
  const hipError_t e = tb::launch_act8_prep(static_cast<const uint16_t*>(x), g.B, g.K, const_cast<uint8_t*>(g.act),
                                            stream);
  if (e != hipSuccess) return TB_ERR_LAUNCH;
  return launched(tb::launch_gemv_multi(&g, 1, stream));
}

// One dense GEMV call with its activations as bf16 x' (encoded as the act8
// operand into `workspace`, then the product) or as the act8 operand itself
// (one launch; the workspace is not used).
tb_status gemv_call(const void* x, int x_dtype, int64_t B, const uint32_t* codes, const uint16_t* scales, int64_t N,
                    int64_t K, float* y, void* workspace, size_t workspace_bytes, int64_t planes, hipStream_t stream) {
  if (x_dtype != TB_BF16 && x_dtype != TB_ACT8) return TB_ERR_DTYPE;
  if (x_dtype == TB_ACT8) {
    const tb_gemv_segment g{static_cast<const uint8_t*>(x), B, codes, scales, N, K, y, planes, 1};
    const tb_status st = check_gemv(g);
    if (st != TB_OK || B == 0) return st;
    return launched(tb::launch_gemv_multi(&g, 1, stream));
  }
  const tb_gemv_segment g{static_cast<const uint8_t*>(workspace), B, codes, scales, N, K, y, planes, 1};
  const tb_status st = check_gemv_bf16(x, g);
  if (st != TB_OK || B == 0) return st;
  const size_t ab = act8_bytes((size_t)B * (size_t)K);
  if (!workspace || workspace_bytes < ab) return TB_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TB_ERR_ALIGN;
  if (overlap(workspace, ab, x, (size_t)B * (size_t)K * 2) || overlap(workspace, ab, codes, gemv_code_bytes(g)) ||
      overlap(workspace, ab, scales, gemv_scale_bytes(g)) || overlap(workspace, ab, y, (size_t)B * (size_t)N * 4))
    return TB_ERR_ALIAS;
  return encode_and_multiply(x, g, stream);
}

// ---------------------------------------------------------------- no-alloc GEMV
// tb_ternary_gemv_noalloc encodes its activations into this library-owned
// array instead of a caller workspace.  Host code never passes `scratch`
// itself to a kernel (on the host the name is a stand-in, not the device
// address): the device address is looked up once per device, with that device
// current, and kept here.
static __device__ __align__(256) unsigned char scratch[TB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null until looked up)

// The device address of `scratch` on the current device.
tb_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TB_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TB_ERR_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return TB_OK;
}

// arguments of the GEMM entry points that take a workspace (NULL allowed)
tb_status check_gemm_ws(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales, int64_t N,
                        int64_t K, const void* y, int y_dtype, const float* workspace, size_t workspace_bytes) {
  if (!dtype_ok(y_dtype)) return TB_ERR_DTYPE;
  if (!dims_ok(N, K) || K > TB_GEMM_MAX_K || M < 0 || M > (int64_t)65535 * 128) return TB_ERR_SHAPE;
  if (M == 0) return TB_OK;
  if (!x || !codes || !scales || !y) return TB_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned16(y) || (workspace && !aligned16(workspace)))
    return TB_ERR_ALIGN;
  const size_t nk = (size_t)N * (size_t)K, yb = (size_t)M * (size_t)N * dtype_bytes(y_dtype);
  if (overlap(y, yb, x, (size_t)M * K * 2) || overlap(y, yb, codes, nk / 4) || overlap(y, yb, scales, nk / 64))
    return TB_ERR_ALIAS;
  const size_t wb = workspace ? workspace_bytes : 0;
  if (overlap(workspace, wb, x, (size_t)M * K * 2) || overlap(workspace, wb, codes, nk / 4) ||
      overlap(workspace, wb, scales, nk / 64) || overlap(workspace, wb, y, yb))
    return TB_ERR_ALIAS;
  return TB_OK;
}

}  // namespace

extern "C" {

const char* tb_status_string(int status) {
  switch (status) {
    case TB_OK: return "TB_OK";
    case TB_ERR_NULL: return "TB_ERR_NULL: a required pointer is NULL";
    case TB_ERR_SHAPE: return "TB_ERR_SHAPE: N and K must be positive multiples of 128 and the batch in range";
    case TB_ERR_ALIGN: return "TB_ERR_ALIGN: pointers must be 16-byte aligned";
    case TB_ERR_DTYPE: return "TB_ERR_DTYPE: unknown dtype";
    case TB_ERR_FORMAT: return "TB_ERR_FORMAT: unknown format or wrong planes for it";
    case TB_ERR_LAUNCH: return "TB_ERR_LAUNCH: the HIP runtime refused the launch";
    case TB_ERR_UNSUPPORTED: return "TB_ERR_UNSUPPORTED: not implemented";
    case TB_ERR_ALIAS: return "TB_ERR_ALIAS: output overlaps an input";
    case TB_ERR_WORKSPACE: return "TB_ERR_WORKSPACE: the workspace is missing or smaller than the call needs";
    default: return "unknown tb_status";
  }
}

int tb_version(void) { return 300; }

size_t tb_act8_bytes(int64_t B, int64_t K) {
  if (B < 0 || K <= 0 || K % kGroup) return 0;
  return act8_bytes((size_t)B * (size_t)K);
}

// The 2:4 format stores whole blocks of four 128-groups: N * K' elements'
// worth of planes for K' = K rounded up to a multiple of 512.
static size_t nk24(int64_t N, int64_t K) { return (size_t)N * (size_t)((K + 511) / 512 * 512); }

tb_status tb_packed_bytes(int fmt, int64_t N, int64_t K, size_t* code_bytes, size_t* meta_bytes,
                          size_t* scale_bytes) {
  if (fmt != TB_FMT_DENSE && fmt != TB_FMT_24 && fmt != TB_FMT_DENSE_MINERR && fmt != TB_FMT_DENSE_RESID)
    return TB_ERR_FORMAT;
  if (!dims_ok(N, K)) return TB_ERR_SHAPE;
  const size_t nk = fmt == TB_FMT_24 ? nk24(N, K) : (size_t)N * (size_t)K;
  const size_t planes = fmt == TB_FMT_DENSE_RESID ? 2 : 1;
  if (code_bytes) *code_bytes = fmt == TB_FMT_24 ? nk / 16 : planes * nk / 4;
  if (meta_bytes) *meta_bytes = fmt == TB_FMT_24 ? nk / 8 : 0;
  if (scale_bytes) *scale_bytes = planes * nk / 64;
  return TB_OK;
}

tb_status tb_fwht128(const void* x, int x_dtype, void* y, int y_dtype, int64_t rows, int64_t K, void* stream) {
  const tb_status st = check_fwht(x, x_dtype, y, y_dtype, rows, K);
  if (st != TB_OK || rows == 0) return st;
  return launched(tb::launch_fwht128(x, x_dtype, y, y_dtype, rows, K, as_stream(stream)));
}

tb_status tb_fwht128_multi(const tb_fwht_segment* segs, int count, void* stream) {
  if (count < 0 || count > TB_MAX_SEGMENTS) return TB_ERR_SHAPE;
  if (count == 0) return TB_OK;
  if (!segs) return TB_ERR_NULL;
  tb_fwht_segment live[TB_MAX_SEGMENTS];
  int n = 0;
  for (int c = 0; c < count; ++c) {
    const tb_fwht_segment& a = segs[c];
    if (a.reserved != 0 || a.x_parts < 0 || a.x_parts > TB_MAX_PARTS) return TB_ERR_SHAPE;
    const int ap = a.x_parts > 1 ? a.x_parts : 1;
    if (ap > 1 && a.x_dtype != TB_F32) return TB_ERR_DTYPE;
    const tb_status st = check_fwht(a.x, a.x_dtype, a.y, a.y_dtype, a.rows, a.K);
    if (st != TB_OK) return st;
    // the partial inputs may not be overwritten while other lanes still read them
    if (ap > 1 && a.rows > 0 &&
        overlap(a.x, ap * fwht_in_bytes(a.rows, a.K, a.x_dtype), a.y, fwht_out_bytes(a.rows, a.K, a.y_dtype)))
      return TB_ERR_ALIAS;
    for (int d = 0; d < c; ++d) {
      const tb_fwht_segment& b = segs[d];
      if (a.rows == 0 || b.rows == 0) continue;
      const int bp = b.x_parts > 1 ? b.x_parts : 1;
      const size_t ai = ap * fwht_in_bytes(a.rows, a.K, a.x_dtype), ao = fwht_out_bytes(a.rows, a.K, a.y_dtype);
      const size_t bi = bp * fwht_in_bytes(b.rows, b.K, b.x_dtype), bo = fwht_out_bytes(b.rows, b.K, b.y_dtype);
      if (overlap(a.y, ao, b.y, bo) || overlap(a.y, ao, b.x, bi) || overlap(b.y, bo, a.x, ai)) return TB_ERR_ALIAS;
    }
    if (a.rows > 0) live[n++] = a;
  }
  if (n == 0) return TB_OK;
  return launched(tb::launch_fwht128_multi(live, n, as_stream(stream)));
}

tb_status tb_quantize_pack(const float* W, int64_t N, int64_t K, int fmt, uint32_t* codes, uint32_t* meta,
                           uint16_t* scales, int32_t* err_flag, void* stream) {
  if (fmt != TB_FMT_DENSE && fmt != TB_FMT_24 && fmt != TB_FMT_DENSE_MINERR && fmt != TB_FMT_DENSE_RESID)
    return TB_ERR_FORMAT;
  if (fmt != TB_FMT_24 && meta) return TB_ERR_FORMAT;
  if (!dims_ok(N, K)) return TB_ERR_SHAPE;
  if (!W || !codes || !scales || (fmt == TB_FMT_24 && !meta)) return TB_ERR_NULL;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(scales) || (meta && !aligned16(meta))) return TB_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(err_flag) & 3u) != 0) return TB_ERR_ALIGN;
  const size_t nk = (size_t)N * (size_t)K, nkp = nk24(N, K);
  const bool dense = fmt != TB_FMT_24;
  const size_t planes = fmt == TB_FMT_DENSE_RESID ? 2 : 1;
  const size_t cb = dense ? planes * nk / 4 : nkp / 16, mb = dense ? 0 : nkp / 8,
               sb = dense ? planes * nk / 64 : nkp / 64;
  if (overlap(W, nk * 4, codes, cb) || overlap(W, nk * 4, scales, sb) || overlap(codes, cb, scales, sb) ||
      (meta && (overlap(W, nk * 4, meta, mb) || overlap(meta, mb, codes, cb) || overlap(meta, mb, scales, sb))))
    return TB_ERR_ALIAS;
  return launched(tb::launch_quantize128(W, N, K, fmt, codes, meta, scales, err_flag, as_stream(stream)));
}

tb_status tb_act8_prep(const uint16_t* x, int64_t B, int64_t K, uint8_t* act, void* stream) {
  if (B < 0 || K <= 0 || K % kGroup) return TB_ERR_SHAPE;
  if (B == 0) return TB_OK;
  if (!x || !act) return TB_ERR_NULL;
  if (!aligned16(x) || !aligned16(act)) return TB_ERR_ALIGN;
  const size_t n = (size_t)B * (size_t)K;
  if (overlap(x, n * 2, act, act8_bytes(n))) return TB_ERR_ALIAS;
  return launched(tb::launch_act8_prep(x, B, K, act, as_stream(stream)));
}

tb_status tb_ternary_gemv(const void* x, int x_dtype, int64_t B, const uint32_t* codes, const uint16_t* scales,
                          int64_t N, int64_t K, float* y, void* workspace, size_t workspace_bytes, void* stream) {
  return gemv_call(x, x_dtype, B, codes, scales, N, K, y, workspace, workspace_bytes, 1, as_stream(stream));
}

tb_status tb_ternary_gemv_noalloc(const uint16_t* x, int64_t B, const uint32_t* codes, const uint16_t* scales,
                                  int64_t N, int64_t K, float* y, void* stream) {
  tb_gemv_segment g{nullptr, B, codes, scales, N, K, y, 1, 1};
  tb_status st = check_gemv_bf16(x, g);
  if (st != TB_OK || B == 0) return st;
  if (act8_bytes((size_t)B * (size_t)K) > (size_t)TB_NOALLOC_SCRATCH_BYTES) return TB_ERR_WORKSPACE;
  void* p = nullptr;
  st = scratch_address(&p);
  if (st != TB_OK) return st;
  g.act = static_cast<const uint8_t*>(p);
  return encode_and_multiply(x, g, as_stream(stream));
}

tb_status tb_ternary_gemv_resid(const void* x, int x_dtype, int64_t B, const uint32_t* codes, const uint16_t* scales,
                                int64_t N, int64_t K, float* y, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return gemv_call(x, x_dtype, B, codes, scales, N, K, y, workspace, workspace_bytes, 2, as_stream(stream));
}

tb_status tb_ternary_gemv_multi(const tb_gemv_segment* segs, int count, void* stream) {
  if (count < 0 || count > TB_MAX_SEGMENTS) return TB_ERR_SHAPE;
  if (count == 0) return TB_OK;
  if (!segs) return TB_ERR_NULL;
  tb_gemv_segment live[TB_MAX_SEGMENTS];
  int n = 0;
  for (int c = 0; c < count; ++c) {
    const tb_gemv_segment& a = segs[c];
    const tb_status st = check_gemv(a);
    if (st != TB_OK) return st;
    if (a.B == 0) continue;
    const size_t ay = gemv_y_bytes(a);
    for (int d = 0; d < count; ++d) {
      const tb_gemv_segment& b = segs[d];
      if (d == c || b.B == 0) continue;
      if (overlap(a.y, ay, b.act, act8_bytes((size_t)b.B * b.K)) || overlap(a.y, ay, b.codes, gemv_code_bytes(b)) ||
          overlap(a.y, ay, b.scales, gemv_scale_bytes(b)) || (d < c && overlap(a.y, ay, b.y, gemv_y_bytes(b))))
        return TB_ERR_ALIAS;
    }
    live[n] = a;
    live[n].planes = gemv_planes(a);
    live[n++].parts = gemv_parts(a);
  }
  if (n == 0) return TB_OK;
  return launched(tb::launch_gemv_multi(live, n, as_stream(stream)));
}

// the arguments of one 2:4 product, without the launch
static tb_status check_gemv24(const tb_gemv24_segment& a) {
  if (!dims_ok(a.N, a.K) || a.B < 0 || a.B > TB_GEMV_MAX_BATCH) return TB_ERR_SHAPE;
  if (a.B == 0) return TB_OK;
  if (!a.x || !a.meta || !a.signs || !a.scales || !a.y) return TB_ERR_NULL;
  if (!aligned16(a.x) || !aligned16(a.meta) || !aligned16(a.signs) || !aligned16(a.scales) || !aligned16(a.y))
    return TB_ERR_ALIGN;
  return TB_OK;
}

// does y of segment a overlap any input (or, with with_y, the output) of b
static bool gemv24_y_overlaps(const tb_gemv24_segment& a, const tb_gemv24_segment& b, bool with_y) {
  const size_t yb = (size_t)a.B * (size_t)a.N * 4, nk = nk24(b.N, b.K);
  return overlap(a.y, yb, b.x, (size_t)b.B * b.K * 2) || overlap(a.y, yb, b.meta, nk / 8) ||
         overlap(a.y, yb, b.signs, nk / 16) || overlap(a.y, yb, b.scales, nk / 64) ||
         (with_y && overlap(a.y, yb, b.y, (size_t)b.B * (size_t)b.N * 4));
}

tb_status tb_ternary24_gemv(const uint16_t* x, int64_t B, const uint32_t* meta, const uint32_t* signs,
                            const uint16_t* scales, int64_t N, int64_t K, float* y, void* stream) {
  const tb_gemv24_segment a{x, meta, signs, scales, y, B, N, K};
  const tb_status st = check_gemv24(a);
  if (st != TB_OK || B == 0) return st;
  if (gemv24_y_overlaps(a, a, false)) return TB_ERR_ALIAS;
  return launched(tb::launch_gemv_ternary24(x, B, meta, signs, scales, N, K, y, as_stream(stream)));
}

tb_status tb_ternary24_gemv_multi(const tb_gemv24_segment* segs, int count, void* stream) {
  if (count < 0 || count > TB_MAX_SEGMENTS) return TB_ERR_SHAPE;
  if (count == 0) return TB_OK;
  if (!segs) return TB_ERR_NULL;
  tb_gemv24_segment live[TB_MAX_SEGMENTS];
  int n = 0;
  for (int c = 0; c < count; ++c) {
    const tb_status st = check_gemv24(segs[c]);
    if (st != TB_OK) return st;
    if (segs[c].B == 0) continue;
    for (int d = 0; d < count; ++d)
      if (segs[d].B != 0 && gemv24_y_overlaps(segs[c], segs[d], d != c)) return TB_ERR_ALIAS;
    live[n++] = segs[c];
  }
  if (n == 0) return TB_OK;
  return launched(tb::launch_gemv24_multi(live, n, as_stream(stream)));
}

// the arguments of one GEMM product, without the launch
static tb_status check_gemm(const tb_gemm_segment& a) {
  if (!dtype_ok(a.y_dtype)) return TB_ERR_DTYPE;
  if (!dims_ok(a.N, a.K) || a.K > TB_GEMM_MAX_K || a.M < 0 || a.M > (int64_t)65535 * 128 || a.reserved != 0)
    return TB_ERR_SHAPE;
  if (a.M == 0) return TB_OK;
  if (!a.x || !a.codes || !a.scales || !a.y) return TB_ERR_NULL;
  if (!aligned16(a.x) || !aligned16(a.codes) || !aligned16(a.scales) || !aligned16(a.y)) return TB_ERR_ALIGN;
  return TB_OK;
}

// does y of product a overlap any input (or, with with_y, the output) of b
static bool gemm_y_overlaps(const tb_gemm_segment& a, const tb_gemm_segment& b, bool with_y) {
  const size_t yb = (size_t)a.M * (size_t)a.N * dtype_bytes(a.y_dtype), nk = (size_t)b.N * (size_t)b.K;
  return overlap(a.y, yb, b.x, (size_t)b.M * b.K * 2) || overlap(a.y, yb, b.codes, nk / 4) ||
         overlap(a.y, yb, b.scales, nk / 64) ||
         (with_y && overlap(a.y, yb, b.y, (size_t)b.M * (size_t)b.N * dtype_bytes(b.y_dtype)));
}

tb_status tb_ternary_gemm(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales, int64_t N,
                          int64_t K, void* y, int y_dtype, void* stream) {
  const tb_gemm_segment a{x, codes, scales, y, M, N, K, y_dtype, 0};
  const tb_status st = check_gemm(a);
  if (st != TB_OK || M == 0) return st;
  if (gemm_y_overlaps(a, a, false)) return TB_ERR_ALIAS;
  return launched(tb::launch_gemm_ternary(x, M, codes, scales, N, K, y, y_dtype, as_stream(stream)));
}

tb_status tb_ternary_gemm_multi(const tb_gemm_segment* segs, int count, void* stream) {
  if (count < 0 || count > TB_MAX_SEGMENTS) return TB_ERR_SHAPE;
  if (count == 0) return TB_OK;
  if (!segs) return TB_ERR_NULL;
  tb_gemm_segment live[TB_MAX_SEGMENTS];
  int n = 0;
  bool skinny = true;
  for (int c = 0; c < count; ++c) {
    const tb_status st = check_gemm(segs[c]);
    if (st != TB_OK) return st;
    if (segs[c].M == 0) continue;
    for (int d = 0; d < count; ++d)
      if (segs[d].M != 0 && gemm_y_overlaps(segs[c], segs[d], d != c)) return TB_ERR_ALIAS;
    skinny = skinny && segs[c].M <= tb::kSkinnyMaxRows;
    live[n++] = segs[c];
  }
  if (n == 0) return TB_OK;
  const hipStream_t st = as_stream(stream);
  if (skinny) return launched(tb::launch_gemm_skinny_multi(live, n, st));
  for (int c = 0; c < n; ++c) {
    const tb_gemm_segment& a = live[c];
    const tb_status r = launched(tb::launch_gemm_ternary(static_cast<const uint16_t*>(a.x), a.M, a.codes, a.scales,
                                                         a.N, a.K, a.y, a.y_dtype, st));
    if (r != TB_OK) return r;
  }
  return TB_OK;
}

size_t tb_ternary_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K) {
  if (!dims_ok(N, K) || K > TB_GEMM_MAX_K || M <= 0 || M > (int64_t)65535 * 128) return 0;
  const int S = tb::gemm_splitk_parts(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

tb_status tb_ternary_gemm_splitk(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                 int64_t N, int64_t K, void* y, int y_dtype, float* workspace,
                                 size_t workspace_bytes, void* stream) {
  const tb_status st = check_gemm_ws(x, M, codes, scales, N, K, y, y_dtype, workspace, workspace_bytes);
  if (st != TB_OK || M == 0) return st;
  return launched(tb::launch_gemm_ternary_splitk(x, M, codes, scales, N, K, y, y_dtype, workspace,
                                                 workspace ? workspace_bytes : 0, false, as_stream(stream)));
}

tb_status tb_ternary_gemm_rotated(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                  int64_t N, int64_t K, void* y, int y_dtype, float* workspace,
                                  size_t workspace_bytes, void* stream) {
  const tb_status st = check_gemm_ws(x, M, codes, scales, N, K, y, y_dtype, workspace, workspace_bytes);
  if (st != TB_OK || M == 0) return st;
  return launched(tb::launch_gemm_ternary_splitk(x, M, codes, scales, N, K, y, y_dtype, workspace,
                                                 workspace ? workspace_bytes : 0, true, as_stream(stream)));
}

}  // extern "C"
