"""Thin ctypes binding over libtb.so (the C ABI declared in include/tb.h).

Argument marshalling only: tensors are device buffers (torch is used for
device memory and streams), every step of the computation runs in the HIP
kernels behind the C ABI.  There is no fallback: if the library is missing or
a call fails, these functions raise.

Dtypes on the Python side (bit patterns are what matter):
  activations x      torch.bfloat16 (or int16/uint16 bit views)  [rows, K]
  act8 operand       torch.uint8, flat, exactly tb_act8_bytes(B, K) bytes
  weights W          torch.float32 [N, K]
  codes              torch.int32 (uint32 bit patterns): dense [N/16, K/128, 128],
                     2:4 sign plane [N/16, G4, 64, 2] (G4 = ceil(K/512))
  meta               torch.int32, 2:4 only: [N/16, G4, 64, 4]
  scales             torch.float16 (fp16 bit patterns), tile-major: [N/16, K/128, 16]
                     (two-plane [N/16, 2K/128, 16]; 2:4 [N/16, G4, 4, 4, 4])
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtb.so")

TB_F32, TB_BF16, TB_ACT8 = 0, 1, 2
TB_FMT_DENSE, TB_FMT_24, TB_FMT_DENSE_MINERR, TB_FMT_DENSE_RESID = 0, 1, 2, 3
TB_EFLAG_NONFINITE, TB_EFLAG_SCALE_OVF = 1, 2
TB_GEMV_MAX_BATCH = 16
TB_MAX_SEGMENTS = 8
TB_NOALLOC_SCRATCH_BYTES = 4 << 20

_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_int = ctypes.c_int

class FwhtSegment(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("rows", ctypes.c_int64), ("K", ctypes.c_int64),
                ("x_dtype", ctypes.c_int), ("y_dtype", ctypes.c_int), ("x_parts", ctypes.c_int),
                ("reserved", ctypes.c_int)]


class Gemv24Segment(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("signs", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("y", ctypes.c_void_p), ("B", ctypes.c_int64), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64)]


class GemmSegment(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("y_dtype", ctypes.c_int), ("reserved", ctypes.c_int)]


class GemvSegment(ctypes.Structure):
    _fields_ = [("act", ctypes.c_void_p), ("B", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("y", ctypes.c_void_p),
                ("planes", ctypes.c_int64), ("parts", ctypes.c_int64)]


SIGNATURES = {
    "tb_status_string": (ctypes.c_char_p, [_int]),
    "tb_version": (_int, []),
    "tb_packed_bytes": (_int, [_int, _i64, _i64, ctypes.POINTER(ctypes.c_size_t),
                               ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "tb_fwht128": (_int, [_vp, _int, _vp, _int, _i64, _i64, _vp]),
    "tb_fwht128_multi": (_int, [ctypes.POINTER(FwhtSegment), _int, _vp]),
    "tb_ternary_gemv_multi": (_int, [ctypes.POINTER(GemvSegment), _int, _vp]),
    "tb_quantize_pack": (_int, [_vp, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp]),
    "tb_ternary_gemv": (_int, [_vp, _int, _i64, _vp, _vp, _i64, _i64, _vp, _vp, ctypes.c_size_t, _vp]),
    "tb_ternary_gemv_noalloc": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _vp, _vp]),
    "tb_ternary_gemv_resid": (_int, [_vp, _int, _i64, _vp, _vp, _i64, _i64, _vp, _vp, ctypes.c_size_t, _vp]),
    "tb_act8_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "tb_act8_prep": (_int, [_vp, _i64, _i64, _vp, _vp]),
    "tb_ternary24_gemv": (_int, [_vp, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _vp]),
    "tb_ternary24_gemv_multi": (_int, [ctypes.POINTER(Gemv24Segment), _int, _vp]),
    "tb_ternary_gemm": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _vp, _int, _vp]),
    "tb_ternary_gemm_multi": (_int, [ctypes.POINTER(GemmSegment), _int, _vp]),
    "tb_ternary_gemm_splitk_workspace": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "tb_ternary_gemm_splitk": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _vp, _int, _vp, ctypes.c_size_t, _vp]),
    "tb_ternary_gemm_rotated": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _vp, _int, _vp, ctypes.c_size_t, _vp]),
}


class TBError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {status_string(code)}")


def lib():
    """Load libtb.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m ternary_weights_hadamard_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(code):
    return lib().tb_status_string(int(code)).decode()


def _check(code, where):
    if code != 0:
        raise TBError(code, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t):
    if t.dtype == torch.float32:
        return TB_F32
    if t.dtype == torch.uint8:
        return TB_ACT8
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return TB_BF16
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("buffers must be contiguous device tensors")


def tb_packed_bytes(fmt, n, k):
    c, m, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().tb_packed_bytes(int(fmt), int(n), int(k), ctypes.byref(c), ctypes.byref(m), ctypes.byref(s)),
           "tb_packed_bytes")
    return c.value, m.value, s.value


def tb_act8_bytes(b, k):
    return int(lib().tb_act8_bytes(int(b), int(k)))


def tb_fwht128(x, y=None, out_dtype=None, stream=None):
    """y[r, 128b + i] = sum_j H[i, j] / sqrt(128) * x[r, 128b + j]; y may be x.
    out_dtype torch.uint8 (or a uint8 y) writes the act8 GEMV operand instead."""
    _dev(x)
    rows = x.numel() // x.shape[-1] if x.numel() else 0
    if y is None:
        if out_dtype == torch.uint8:
            y = torch.empty(tb_act8_bytes(rows, x.shape[-1]), dtype=torch.uint8, device=x.device)
        else:
            y = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _dev(y)
    _check(lib().tb_fwht128(_p(x), _dt(x), _p(y), _dt(y), rows, x.shape[-1], _stream(stream)), "tb_fwht128")
    return y


def tb_fwht128_multi(pairs, stream=None):
    """One launch rotating several arrays: pairs = [(x, y), ...] or
    [(x, y, x_parts), ...], each with its own dtypes (a uint8 y means the act8
    operand).  With x_parts > 1, x is [x_parts, rows, K] fp32 partial results
    added in order before the transform (y is [rows, K])."""
    if not pairs:
        return
    for p in pairs:
        _dev(p[0], p[1])
    arr = (FwhtSegment * len(pairs))()
    for c, p in enumerate(pairs):
        x, y = p[0], p[1]
        parts = int(p[2]) if len(p) > 2 else 1
        if parts > 1:
            if x.dim() < 2 or x.shape[0] != parts:
                raise ValueError(f"tb_fwht128_multi: x_parts={parts} needs x of shape [{parts}, rows, K], "
                                 f"got {tuple(x.shape)}")
            inner = x[0]
        else:
            inner = x
        rows = inner.numel() // inner.shape[-1] if inner.numel() else 0
        arr[c] = FwhtSegment(x.data_ptr(), y.data_ptr(), rows, x.shape[-1], _dt(x), _dt(y), parts, 0)
    _check(lib().tb_fwht128_multi(arr, len(pairs), _stream(stream)), "tb_fwht128_multi")


def tb_quantize_pack(w, fmt=TB_FMT_DENSE, codes=None, meta=None, scales=None, err_flag=None, stream=None):
    """Quantise fp32 W [N, K]; returns (codes, meta, scales).  For TB_FMT_24 `codes` is the sign plane;
    for TB_FMT_DENSE_RESID codes and scales hold both planes, groups interleaved."""
    _dev(w)
    n, k = w.shape
    dev = w.device
    planes = 2 if fmt == TB_FMT_DENSE_RESID else 1
    g4 = -(-k // 512)  # 2:4 blocks of four groups per tile
    if codes is None:
        shape = (n // 16, planes * k // 128, 128) if fmt != TB_FMT_24 else (n // 16, g4, 64, 2)
        codes = torch.empty(shape, dtype=torch.int32, device=dev)
    if meta is None and fmt == TB_FMT_24:
        meta = torch.empty((n // 16, g4, 64, 4), dtype=torch.int32, device=dev)
    if scales is None:
        shape = (n // 16, planes * k // 128, 16) if fmt != TB_FMT_24 else (n // 16, g4, 4, 4, 4)
        scales = torch.empty(shape, dtype=torch.float16, device=dev)
    _dev(codes, meta, scales, err_flag)
    _check(lib().tb_quantize_pack(_p(w), n, k, int(fmt), _p(codes), _p(meta), _p(scales), _p(err_flag),
                                  _stream(stream)), "tb_quantize_pack")
    return codes, meta, scales


def tb_act8_prep(x, act=None, stream=None):
    """Encode bf16 activations x [B, K] as the act8 operand of tb_ternary_gemv."""
    _dev(x)
    b, k = x.shape
    if act is None:
        act = torch.empty(max(tb_act8_bytes(b, k), 1), dtype=torch.uint8, device=x.device)
    _dev(act)
    _check(lib().tb_act8_prep(_p(x), b, k, _p(act), _stream(stream)), "tb_act8_prep")
    return act


def _act8_operand(act, batch, k, where):
    """Check that `act` is the act8 operand of exactly `batch` rows of length k
    (its scale part starts at byte 4 * batch * k, so the size must match)."""
    if batch is None:
        raise ValueError(f"{where}: an act8 operand needs its batch")
    if batch == 0:
        return  # a no-op call reads nothing
    if act.dtype != torch.uint8 or act.numel() != tb_act8_bytes(batch, k):
        raise ValueError(f"{where}: act8 operand of {batch} rows x {k} must be a uint8 buffer of "
                         f"{tb_act8_bytes(batch, k)} bytes (got {act.dtype}, {act.numel()} elements)")


def _dense_n(scales):
    """Output rows of dense-format scales [N/16, G, 16]."""
    if scales.dim() != 3 or scales.shape[2] != 16:
        raise ValueError(f"dense scales must be [N/16, G, 16] (got {tuple(scales.shape)})")
    return scales.shape[0] * 16


def _gemv(fn, where, x, codes, scales, k, batch, y, workspace, stream):
    _dev(x, codes, scales)
    n = _dense_n(scales)
    if x.dtype == torch.uint8:
        _act8_operand(x, batch, k, where)
        b, dt, wbytes = int(batch), TB_ACT8, 0
    else:
        if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or x.dim() != 2 or x.shape[1] != k:
            raise ValueError(f"{where}: x must be bf16 [B, {k}] (got {x.dtype} {tuple(x.shape)})")
        b, dt = x.shape[0], TB_BF16
        if batch is not None and int(batch) != b:
            raise ValueError(f"{where}: batch {batch} but x has {b} rows")
        if workspace is None:
            workspace = torch.empty(max(tb_act8_bytes(b, k), 16), dtype=torch.uint8, device=x.device)
        wbytes = workspace.numel() * workspace.element_size()
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _dev(y, workspace)
    _check(fn(_p(x), dt, b, _p(codes), _p(scales), n, k, _p(y), _p(workspace) if dt == TB_BF16 else None,
              wbytes, _stream(stream)), where)
    return y


def tb_ternary_gemv(x, codes, scales, batch=None, y=None, workspace=None, stream=None):
    """y[b, n] (fp32) = sum_g scale[n, g] * sum_k t[n, k] x[b, k].  x is either
    the rotated activations as bf16 [B, K] (encoded into `workspace`, a uint8
    device tensor of at least tb_act8_bytes(B, K) bytes, allocated here when
    None) or their act8 operand (uint8, exactly tb_act8_bytes(batch, K) bytes,
    `batch` given)."""
    return _gemv(lib().tb_ternary_gemv, "tb_ternary_gemv", x, codes, scales, scales.shape[1] * 128, batch, y,
                 workspace, stream)


def tb_ternary_gemv_noalloc(x, codes, scales, y, stream=None):
    """tb_ternary_gemv of bf16 x [B, K] into the caller's fp32 y [B, N] with the
    library's own device array for the encoded activations: nothing is
    allocated (the caller passes y).  Calls that may overlap on one GPU race."""
    _dev(x, codes, scales, y)
    n, k = _dense_n(scales), scales.shape[1] * 128
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"tb_ternary_gemv_noalloc: x must be bf16 [B, {k}] (got {x.dtype} {tuple(x.shape)})")
    if y.dtype != torch.float32 or tuple(y.shape) != (x.shape[0], n):
        raise ValueError(f"tb_ternary_gemv_noalloc: y must be float32 [{x.shape[0]}, {n}]")
    _check(lib().tb_ternary_gemv_noalloc(_p(x), x.shape[0], _p(codes), _p(scales), n, k, _p(y), _stream(stream)),
           "tb_ternary_gemv_noalloc")
    return y


def tb_ternary_gemv_resid(x, codes, scales, batch=None, y=None, workspace=None, stream=None):
    """tb_ternary_gemv over two-plane weights (TB_FMT_DENSE_RESID): codes
    [N/16, 2K/128, 128], scales [N, 2K/128], groups of the planes interleaved."""
    return _gemv(lib().tb_ternary_gemv_resid, "tb_ternary_gemv_resid", x, codes, scales, scales.shape[1] // 2 * 128,
                 batch, y, workspace, stream)


def tb_ternary_gemv_multi(segments, stream=None):
    """One launch of several GEMVs: segments = [(act, codes, scales, batch, y[, planes[, parts]]), ...];
    planes is 1 (default) or 2 for two-plane weights; parts > 1 (batch 1) splits K over that many
    workgroups per tile and y receives the parts, [parts, batch, N], whose sum is the product."""
    if not segments:
        return
    arr = (GemvSegment * len(segments))()
    for c, seg in enumerate(segments):
        act, codes, scales, batch, y = seg[:5]
        planes = int(seg[5]) if len(seg) > 5 else 1
        parts = int(seg[6]) if len(seg) > 6 else 1
        _dev(act, codes, scales, y)
        n, g = _dense_n(scales), scales.shape[1]
        k = g // max(planes, 1) * 128
        _act8_operand(act, int(batch), k, "tb_ternary_gemv_multi")
        if y.numel() < max(parts, 1) * int(batch) * n:
            raise ValueError(f"tb_ternary_gemv_multi: y holds {y.numel()} floats, needs {max(parts, 1)} x {batch} x {n}")
        arr[c] = GemvSegment(act.data_ptr(), int(batch), codes.data_ptr(), scales.data_ptr(), n, k, y.data_ptr(),
                             planes, parts)
    _check(lib().tb_ternary_gemv_multi(arr, len(segments), _stream(stream)), "tb_ternary_gemv_multi")


def _planes24(x, meta, signs, scales, where):
    """(B, N, K) of a 2:4 product, its planes checked against x."""
    b, k = x.shape
    n = meta.shape[0] * 16
    g4 = -(-k // 512)
    if tuple(meta.shape) != (n // 16, g4, 64, 4) or tuple(signs.shape) != (n // 16, g4, 64, 2) \
            or scales.numel() != n * g4 * 4:
        raise ValueError(f"{where}: 2:4 planes {tuple(meta.shape)}, {tuple(signs.shape)} do not match K = {k}")
    return b, n, k


def tb_ternary24_gemv(x, meta, signs, scales, y=None, stream=None):
    """x bf16 [B, K]; meta [N/16, G4, 64, 4], signs [N/16, G4, 64, 2], scales
    [N/16, G4, 4, 4, 4] (the stored 2:4 format, G4 = ceil(K/512))."""
    _dev(x, meta, signs, scales)
    b, n, k = _planes24(x, meta, signs, scales, "tb_ternary24_gemv")
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _dev(y)
    _check(lib().tb_ternary24_gemv(_p(x), b, _p(meta), _p(signs), _p(scales), n, k, _p(y), _stream(stream)),
           "tb_ternary24_gemv")
    return y


def tb_ternary24_gemv_multi(segments, stream=None):
    """One launch of several 2:4 GEMVs: segments = [(x, meta, signs, scales, y), ...]
    with the shapes of tb_ternary24_gemv; y fp32 [B, N] each."""
    if not segments:
        return
    arr = (Gemv24Segment * len(segments))()
    for c, (x, meta, signs, scales, y) in enumerate(segments):
        _dev(x, meta, signs, scales, y)
        b, n, k = _planes24(x, meta, signs, scales, "tb_ternary24_gemv_multi")
        if y.numel() < b * n:
            raise ValueError(f"tb_ternary24_gemv_multi: y holds {y.numel()} floats, needs {b} x {n}")
        arr[c] = Gemv24Segment(x.data_ptr(), meta.data_ptr(), signs.data_ptr(), scales.data_ptr(), y.data_ptr(),
                               b, n, k)
    _check(lib().tb_ternary24_gemv_multi(arr, len(segments), _stream(stream)), "tb_ternary24_gemv_multi")


def tb_ternary_gemm(x, codes, scales, y=None, out_dtype=torch.bfloat16, stream=None):
    """Y[m, n] = sum_g scale[n, g] * sum_k t[n, k] x[m, k]; x bf16 [M, K], Y bf16 or fp32."""
    _dev(x, codes, scales)
    m, k = x.shape
    n = _dense_n(scales)
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _dev(y)
    _check(lib().tb_ternary_gemm(_p(x), m, _p(codes), _p(scales), n, k, _p(y), _dt(y), _stream(stream)),
           "tb_ternary_gemm")
    return y


def tb_ternary_gemm_multi(segments, stream=None):
    """Several GEMMs: segments = [(x, codes, scales, y), ...], x bf16 [M, K], y bf16 or fp32 [M, N];
    one launch when every M <= 16, else one launch per product."""
    if not segments:
        return
    arr = (GemmSegment * len(segments))()
    for c, (x, codes, scales, y) in enumerate(segments):
        _dev(x, codes, scales, y)
        m, k = x.shape
        n = _dense_n(scales)
        if y.numel() < m * n:
            raise ValueError(f"tb_ternary_gemm_multi: y holds {y.numel()} elements, needs {m} x {n}")
        arr[c] = GemmSegment(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), y.data_ptr(), m, n, k, _dt(y), 0)
    _check(lib().tb_ternary_gemm_multi(arr, len(segments), _stream(stream)), "tb_ternary_gemm_multi")


def tb_ternary_gemm_splitk_workspace(m, n, k):
    return int(lib().tb_ternary_gemm_splitk_workspace(int(m), int(n), int(k)))


def tb_ternary_gemm_splitk(x, codes, scales, y=None, out_dtype=torch.bfloat16, workspace=None, stream=None):
    """tb_ternary_gemm with K split across workgroups for few activation rows;
    `workspace` is a device tensor of at least tb_ternary_gemm_splitk_workspace
    bytes (allocated here when None)."""
    _dev(x, codes, scales)
    m, k = x.shape
    n = _dense_n(scales)
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    if workspace is None:
        nbytes = tb_ternary_gemm_splitk_workspace(m, n, k)
        workspace = torch.empty(max(nbytes // 4, 4), dtype=torch.float32, device=x.device)
    _dev(y, workspace)
    _check(lib().tb_ternary_gemm_splitk(_p(x), m, _p(codes), _p(scales), n, k, _p(y), _dt(y), _p(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)),
           "tb_ternary_gemm_splitk")
    return y


def tb_ternary_gemm_rotated(x, codes, scales, y=None, out_dtype=torch.bfloat16, workspace=None, stream=None):
    """The GEMM with its output rotated back along N (y = R_N y') in the same
    launch; `workspace` (a device tensor, or None for one pass over K) as in
    tb_ternary_gemm_splitk."""
    _dev(x, codes, scales)
    m, k = x.shape
    n = _dense_n(scales)
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _dev(y, workspace)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().tb_ternary_gemm_rotated(_p(x), m, _p(codes), _p(scales), n, k, _p(y), _dt(y), _p(workspace),
                                         wbytes, _stream(stream)), "tb_ternary_gemm_rotated")
    return y
