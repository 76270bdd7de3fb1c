"""CPU tests of the C ABI: the built library loads, exports every entry point
that include/tb.h declares, and rejects bad arguments on the host before any
GPU work (no call here gets past validation, so no GPU is needed)."""

import ctypes
import os
import re

import pytest

from ternary_weights_hadamard_amd import tb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tb.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tb.LIB_PATH), reason="libtb.so not built")

A = 0x10000  # 16-byte aligned fake device addresses (never dereferenced)
B = 0x20000
C = 0x30000
D = 0x40000
MIS = 0x10008  # 8-byte aligned only


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(tb_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"tb_fwht128", "tb_quantize_pack", "tb_ternary_gemv", "tb_ternary24_gemv", "tb_ternary_gemm"} <= set(names)
    handle = ctypes.CDLL(tb.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert set(names) == set(tb.SIGNATURES), "binding and header disagree"


PROBE_HEADER = os.path.join(ROOT, "include", "tb_probe.h")
PROBE_LIB = os.path.join(os.path.dirname(tb.LIB_PATH), "libtb_probe.so")


@pytest.mark.skipif(not os.path.exists(PROBE_LIB), reason="libtb_probe.so not built")
def test_probe_library_exports_and_validates():
    names = sorted(set(re.findall(r"\b(tbp_[a-z0-9_]+)\s*\(", open(PROBE_HEADER).read())))
    assert names == ["tbp_mfma_bf16", "tbp_stream_read"]
    L = ctypes.CDLL(PROBE_LIB)
    for n in names:
        assert hasattr(L, n), n
    L.tbp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.tbp_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    invalid = 1  # hipErrorInvalidValue, returned before any HIP call
    assert L.tbp_stream_read(None, 4096, _v(B), 1, None) == invalid
    assert L.tbp_stream_read(_v(A), 4096, None, 1, None) == invalid
    assert L.tbp_stream_read(_v(A), 4000, _v(B), 1, None) == invalid      # not a multiple of 4096
    assert L.tbp_stream_read(_v(MIS), 4096, _v(B), 1, None) == invalid    # not 16-byte aligned
    assert L.tbp_stream_read(_v(A), 4096, _v(B), 0, None) == invalid
    assert L.tbp_mfma_bf16(None, 10, 1, None) == invalid
    assert L.tbp_mfma_bf16(_v(B), 0, 1, None) == invalid
    assert L.tbp_mfma_bf16(_v(B), 10, 0, None) == invalid


def test_status_strings_and_version():
    L = tb.lib()
    assert L.tb_version() >= 100
    for code in range(10):
        assert L.tb_status_string(code)
    assert b"WORKSPACE" in L.tb_status_string(9)
    assert b"unknown" in L.tb_status_string(99)


def test_packed_bytes():
    assert tb.tb_packed_bytes(tb.TB_FMT_DENSE, 5120, 17408) == (5120 * 17408 // 4, 0, 5120 * 17408 // 64)
    assert tb.tb_packed_bytes(tb.TB_FMT_24, 17408, 5120) == (17408 * 5120 // 16, 17408 * 5120 // 8, 17408 * 5120 // 64)
    # 2:4 stores whole blocks of four 128-groups: K = 384 takes the room of 512
    assert tb.tb_packed_bytes(tb.TB_FMT_24, 256, 384) == (256 * 512 // 16, 256 * 512 // 8, 256 * 512 // 64)
    assert tb.tb_packed_bytes(tb.TB_FMT_DENSE_MINERR, 256, 384) == tb.tb_packed_bytes(tb.TB_FMT_DENSE, 256, 384)
    assert tb.tb_packed_bytes(tb.TB_FMT_DENSE_RESID, 5120, 5120) == (5120 * 5120 // 2, 0, 5120 * 5120 // 32)
    L = tb.lib()
    assert L.tb_packed_bytes(7, 128, 128, None, None, None) == 5
    assert L.tb_packed_bytes(0, 100, 128, None, None, None) == 2
    assert L.tb_packed_bytes(0, 128, 0, None, None, None) == 2


def _v(x):
    return ctypes.c_void_p(x)


def test_fwht_validation():
    L = tb.lib()
    s = None
    assert L.tb_fwht128(_v(A), 5, _v(B), 1, 1, 128, s) == 4       # unknown dtype
    assert L.tb_fwht128(_v(A), 1, _v(B), 1, 1, 100, s) == 2      # K not a multiple of 128
    assert L.tb_fwht128(_v(A), 1, _v(B), 1, -1, 128, s) == 2     # negative rows
    assert L.tb_fwht128(None, 1, _v(B), 1, 1, 128, s) == 1       # NULL
    assert L.tb_fwht128(_v(MIS), 1, _v(B), 1, 1, 128, s) == 3    # misaligned
    assert L.tb_fwht128(_v(A), 1, _v(A + 64), 1, 1, 128, s) == 8  # partial overlap
    assert L.tb_fwht128(_v(A), 1, _v(A), 0, 1, 128, s) == 8      # in place with different dtypes
    assert L.tb_fwht128(None, 1, None, 1, 0, 128, s) == 0        # empty batch is a no-op
    assert L.tb_fwht128(_v(A), 2, _v(B), 1, 1, 128, s) == 4      # act8 is an output-only dtype
    # act8 output: 4.125 bytes per element, so a y starting 512 bytes after a
    # 256-byte bf16 x does not overlap it, one starting inside x does
    assert L.tb_fwht128(_v(A), 1, _v(A + 128), 2, 1, 128, s) == 8
    assert L.tb_fwht128(_v(A), 2, _v(A), 2, 1, 128, s) == 4


def test_act8_bytes_and_prep_validation():
    L = tb.lib()
    s = None
    assert tb.tb_act8_bytes(1, 5120) == 4 * 5120 + 5120 // 8
    assert tb.tb_act8_bytes(3, 128) == 3 * (4 * 128 + 16)
    assert tb.tb_act8_bytes(0, 128) == 0
    assert tb.tb_act8_bytes(1, 100) == 0 and tb.tb_act8_bytes(-1, 128) == 0
    assert L.tb_act8_prep(_v(A), 1, 100, _v(B), s) == 2
    assert L.tb_act8_prep(_v(A), -1, 128, _v(B), s) == 2
    assert L.tb_act8_prep(None, 1, 128, _v(B), s) == 1
    assert L.tb_act8_prep(_v(A), 1, 128, _v(MIS), s) == 3
    assert L.tb_act8_prep(_v(A), 1, 128, _v(A + 16), s) == 8    # act over x
    assert L.tb_act8_prep(None, 0, 128, None, s) == 0           # empty batch


def test_quantize_validation():
    L = tb.lib()
    s = None
    assert L.tb_quantize_pack(_v(A), 128, 128, 4, _v(B), None, _v(C), None, s) == 5   # bad format
    assert L.tb_quantize_pack(_v(A), 128, 128, 3, _v(B), _v(D), _v(C), None, s) == 5  # meta given for two planes
    # two planes: codes take 8 KB for 128 x 128, so scales 4 KB after them overlap
    # (one plane would end there; that case is not called: it would launch)
    assert L.tb_quantize_pack(_v(A), 128, 128, 3, _v(B), None, _v(B + 4096), None, s) == 8
    assert L.tb_quantize_pack(_v(A), 128, 128, 0, _v(B), _v(D), _v(C), None, s) == 5  # meta given for dense
    assert L.tb_quantize_pack(_v(A), 128, 128, 1, _v(B), None, _v(C), None, s) == 1   # meta missing for 2:4
    assert L.tb_quantize_pack(_v(A), 130, 128, 0, _v(B), None, _v(C), None, s) == 2
    assert L.tb_quantize_pack(_v(A), 128, 0, 0, _v(B), None, _v(C), None, s) == 2
    assert L.tb_quantize_pack(None, 128, 128, 0, _v(B), None, _v(C), None, s) == 1
    assert L.tb_quantize_pack(_v(A), 128, 128, 0, _v(MIS), None, _v(C), None, s) == 3
    assert L.tb_quantize_pack(_v(A), 128, 128, 0, _v(B), None, _v(C), _v(D + 2), s) == 3  # flag misaligned
    assert L.tb_quantize_pack(_v(A), 128, 128, 0, _v(A + 1024), None, _v(C), None, s) == 8  # codes inside W


ACT8, BF16 = tb.TB_ACT8, tb.TB_BF16


def test_gemv_resid_validation():
    L = tb.lib()
    s = None
    R = L.tb_ternary_gemv_resid
    assert R(_v(A), ACT8, 17, _v(B), _v(C), 128, 128, _v(D), None, 0, s) == 2
    assert R(_v(A), ACT8, 1, None, _v(C), 128, 128, _v(D), None, 0, s) == 1
    assert R(_v(A), ACT8, 1, _v(B), _v(C), 128, 128, _v(MIS), None, 0, s) == 3
    assert R(None, ACT8, 0, None, None, 128, 128, None, None, 0, s) == 0
    # y right after one plane's codes (4 KB) overlaps the second plane; after
    # one plane's scales (256 B) overlaps the second plane's scales
    assert R(_v(A), ACT8, 1, _v(B), _v(C), 128, 128, _v(B + 4096), None, 0, s) == 8
    assert R(_v(A), ACT8, 1, _v(B), _v(C), 128, 128, _v(C + 256), None, 0, s) == 8
    # bf16 activations need a workspace of the act8 size
    assert R(_v(A), BF16, 1, _v(B), _v(C), 128, 128, _v(D), None, 0, s) == 9
    assert R(_v(A), BF16, 1, _v(B), _v(C), 128, 128, _v(D), _v(0x50000), 527, s) == 9
    Gs = tb.GemvSegment
    bad_planes = (Gs * 1)(Gs(A, 1, B, C, 128, 128, D, 3))
    assert L.tb_ternary_gemv_multi(bad_planes, 1, s) == 5
    neg_planes = (Gs * 1)(Gs(A, 1, B, C, 128, 128, D, -1))
    assert L.tb_ternary_gemv_multi(neg_planes, 1, s) == 5
    two = (Gs * 2)(Gs(A, 1, B, C, 128, 128, D, 2), Gs(A, 1, B, C, 128, 128, B + 4096, 1))
    assert L.tb_ternary_gemv_multi(two, 2, s) == 8                 # a y inside another's second plane


def test_gemv_validation():
    L = tb.lib()
    s = None
    G = L.tb_ternary_gemv
    # the pre-encoded act8 operand
    assert G(_v(A), ACT8, 17, _v(B), _v(C), 128, 128, _v(D), None, 0, s) == 2   # B > 16
    assert G(_v(A), ACT8, -1, _v(B), _v(C), 128, 128, _v(D), None, 0, s) == 2
    assert G(_v(A), ACT8, 1, _v(B), _v(C), 100, 128, _v(D), None, 0, s) == 2
    assert G(_v(A), ACT8, 1, None, _v(C), 128, 128, _v(D), None, 0, s) == 1
    assert G(_v(A), ACT8, 1, _v(B), _v(C), 128, 128, _v(MIS), None, 0, s) == 3
    assert G(_v(A), ACT8, 1, _v(B), _v(C), 128, 128, _v(B), None, 0, s) == 8     # y over codes
    assert G(_v(A), ACT8, 1, _v(B), _v(C), 128, 128, _v(A + 512), None, 0, s) == 8  # y over act8 (528 bytes)
    assert G(None, ACT8, 0, None, None, 128, 128, None, None, 0, s) == 0         # empty batch
    # dtypes: bf16 x' or the act8 operand only
    assert G(_v(A), tb.TB_F32, 1, _v(B), _v(C), 128, 128, _v(D), None, 0, s) == 4
    assert G(_v(A), 7, 1, _v(B), _v(C), 128, 128, _v(D), None, 0, s) == 4
    # bf16 x': the workspace must hold tb_act8_bytes(B, K) (528 bytes per row of 128)
    W = 0x50000
    assert G(_v(A), BF16, 2, _v(B), _v(C), 128, 128, _v(D), None, 0, s) == 9     # no workspace
    assert G(_v(A), BF16, 2, _v(B), _v(C), 128, 128, _v(D), _v(W), 1055, s) == 9  # one byte short
    assert G(_v(A), BF16, 2, _v(B), _v(C), 128, 128, _v(D), _v(W + 8), 1056, s) == 3  # misaligned workspace
    assert G(_v(MIS), BF16, 2, _v(B), _v(C), 128, 128, _v(D), _v(W), 1056, s) == 3
    assert G(None, BF16, 2, _v(B), _v(C), 128, 128, _v(D), _v(W), 1056, s) == 1
    assert G(_v(A), BF16, 2, _v(B), _v(C), 128, 200, _v(D), _v(W), 1056, s) == 2
    assert G(_v(A), BF16, 2, _v(B), _v(C), 128, 128, _v(A + 256), _v(W), 1056, s) == 8   # y over x (512 B)
    assert G(_v(A), BF16, 2, _v(B), _v(C), 128, 128, _v(D), _v(A + 256), 1056, s) == 8   # workspace over x
    assert G(_v(A), BF16, 2, _v(B), _v(C), 128, 128, _v(D), _v(C), 1056, s) == 8         # workspace over scales
    assert G(_v(A), BF16, 2, _v(B), _v(C), 128, 128, _v(W + 1024), _v(W), 1056, s) == 8  # y over workspace
    assert G(None, BF16, 0, None, None, 128, 128, None, None, 0, s) == 0
    assert L.tb_ternary24_gemv(_v(A), 1, _v(B), None, _v(C), 128, 128, _v(D), s) == 1
    assert L.tb_ternary24_gemv(_v(A), 1, _v(B), _v(C), _v(D), 128, 384, _v(MIS), s) == 3
    assert L.tb_ternary24_gemv(_v(A), 20, _v(B), _v(C), _v(D), 128, 384, _v(A), s) == 2
    # y over the meta plane: 128 x 384 stores whole blocks, 128 x 512 / 8 = 8192 bytes of meta at B
    assert L.tb_ternary24_gemv(_v(A), 1, _v(B), _v(C), _v(D), 128, 384, _v(B + 8192 - 256), s) == 8


def test_grouped_gemm_validation():
    L = tb.lib()
    s = None
    S = tb.GemmSegment
    # x, codes, scales, y, M, N, K, y_dtype, reserved
    two = (S * 2)(S(A, B, C, 0x60000, 16, 128, 128, tb.TB_F32, 0), S(A, B, C, 0x70000, 16, 128, 128, tb.TB_F32, 0))
    assert L.tb_ternary_gemm_multi(two, 9, s) == 2                 # more than TB_MAX_SEGMENTS
    assert L.tb_ternary_gemm_multi(two, -1, s) == 2
    assert L.tb_ternary_gemm_multi(two, 0, s) == 0
    assert L.tb_ternary_gemm_multi(None, 1, s) == 1
    same_y = (S * 2)(S(A, B, C, 0x60000, 16, 128, 128, tb.TB_F32, 0), S(A, B, C, 0x60000, 16, 128, 128, tb.TB_F32, 0))
    assert L.tb_ternary_gemm_multi(same_y, 2, s) == 8              # two products into one y
    y_over_in = (S * 2)(S(A, B, C, 0x60000, 16, 128, 128, tb.TB_F32, 0),
                        S(0x60000, B, C, 0x70000, 16, 128, 128, tb.TB_F32, 0))
    assert L.tb_ternary_gemm_multi(y_over_in, 2, s) == 8           # a y is another's x
    dt = (S * 1)(S(A, B, C, 0x60000, 16, 128, 128, 7, 0))
    assert L.tb_ternary_gemm_multi(dt, 1, s) == 4
    res = (S * 1)(S(A, B, C, 0x60000, 16, 128, 128, tb.TB_F32, 1))
    assert L.tb_ternary_gemm_multi(res, 1, s) == 2                 # reserved must be 0
    mis = (S * 1)(S(A, B, C, MIS, 16, 128, 128, tb.TB_F32, 0))
    assert L.tb_ternary_gemm_multi(mis, 1, s) == 3
    empty = (S * 1)(S(None, None, None, None, 0, 128, 128, tb.TB_F32, 0))
    assert L.tb_ternary_gemm_multi(empty, 1, s) == 0               # M = 0: nothing to do


def test_grouped_24_validation():
    L = tb.lib()
    s = None
    S = tb.Gemv24Segment
    # x, meta, signs, scales, y, B, N, K
    two = (S * 2)(S(A, B, C, D, 0x60000, 1, 128, 128), S(A, B, C, D, 0x61000, 1, 128, 128))
    assert L.tb_ternary24_gemv_multi(two, 9, s) == 2               # more than TB_MAX_SEGMENTS
    assert L.tb_ternary24_gemv_multi(two, -1, s) == 2
    assert L.tb_ternary24_gemv_multi(two, 0, s) == 0
    assert L.tb_ternary24_gemv_multi(None, 1, s) == 1
    same_y = (S * 2)(S(A, B, C, D, 0x60000, 1, 128, 128), S(A, B, C, D, 0x60000, 1, 128, 128))
    assert L.tb_ternary24_gemv_multi(same_y, 2, s) == 8            # two products into one y
    y_over_in = (S * 2)(S(A, B, C, D, 0x60000, 1, 128, 128), S(0x60000, B, C, D, 0x61000, 1, 128, 128))
    assert L.tb_ternary24_gemv_multi(y_over_in, 2, s) == 8         # a y is another's x
    bad = (S * 2)(S(A, B, C, D, 0x60000, 1, 128, 128), S(A, B, C, D, 0x61000, 17, 128, 128))
    assert L.tb_ternary24_gemv_multi(bad, 2, s) == 2               # one bad batch fails the call
    mis = (S * 1)(S(A, B, C, D, MIS, 1, 128, 128))
    assert L.tb_ternary24_gemv_multi(mis, 1, s) == 3
    empty = (S * 1)(S(None, None, None, None, None, 0, 128, 128))
    assert L.tb_ternary24_gemv_multi(empty, 1, s) == 0             # B = 0: nothing to do


def test_grouped_validation():
    L = tb.lib()
    s = None
    F, Gs = tb.FwhtSegment, tb.GemvSegment
    bb = lambda x, y, rows, k: F(x, y, rows, k, tb.TB_BF16, tb.TB_BF16)
    fw = (F * 2)(bb(A, B, 1, 128), bb(C, D, 1, 128))
    assert L.tb_fwht128_multi(fw, 9, s) == 2                       # more than TB_MAX_SEGMENTS
    assert L.tb_fwht128_multi(fw, -1, s) == 2
    assert L.tb_fwht128_multi(fw, 0, s) == 0                       # empty group
    assert L.tb_fwht128_multi(None, 2, s) == 1
    bad_dtype = (F * 2)(bb(A, B, 1, 128), F(C, D, 1, 128, 7, tb.TB_BF16))
    assert L.tb_fwht128_multi(bad_dtype, 2, s) == 4                # one segment's dtype
    act_in = (F * 1)(F(A, B, 1, 128, tb.TB_ACT8, tb.TB_F32))
    assert L.tb_fwht128_multi(act_in, 1, s) == 4                   # act8 is an output-only dtype
    bad = (F * 2)(bb(A, B, 1, 128), bb(C, D, 1, 100))
    assert L.tb_fwht128_multi(bad, 2, s) == 2                      # one bad segment fails the call
    clash = (F * 2)(bb(A, B, 1, 128), bb(C, B + 64, 1, 128))
    assert L.tb_fwht128_multi(clash, 2, s) == 8                    # outputs overlap each other
    reads = (F * 2)(bb(A, B, 1, 128), bb(B, D, 1, 128))
    assert L.tb_fwht128_multi(reads, 2, s) == 8                    # one writes what another reads
    # sizes follow each segment's own dtypes: an fp32 output of 512 bytes at D,
    # and another segment reading bf16 at D + 256 (inside it)
    mixed = (F * 2)(F(A, D, 1, 128, tb.TB_F32, tb.TB_F32), bb(D + 256, C, 1, 128))
    assert L.tb_fwht128_multi(mixed, 2, s) == 8
    gv = (Gs * 2)(Gs(A, 1, B, C, 128, 128, D), Gs(A, 1, B, C, 128, 128, D + 4096))
    assert L.tb_ternary_gemv_multi(gv, 9, s) == 2
    assert L.tb_ternary_gemv_multi(gv, 0, s) == 0
    assert L.tb_ternary_gemv_multi(None, 1, s) == 1
    same_y = (Gs * 2)(Gs(A, 1, B, C, 128, 128, D), Gs(A, 1, B, C, 128, 128, D))
    assert L.tb_ternary_gemv_multi(same_y, 2, s) == 8              # two products into one y
    y_over_in = (Gs * 2)(Gs(A, 1, B, C, 128, 128, D), Gs(D, 1, B, C, 128, 128, D + 4096))
    assert L.tb_ternary_gemv_multi(y_over_in, 2, s) == 8           # a y is another's act
    shape = (Gs * 1)(Gs(A, 17, B, C, 128, 128, D))
    assert L.tb_ternary_gemv_multi(shape, 1, s) == 2


def test_split_gemv_and_summing_rotation_validation():
    # tb_gemv_segment.parts: K split over workgroups, y holding the parts
    L = tb.lib()
    s = None
    F, Gs = tb.FwhtSegment, tb.GemvSegment
    one = lambda *seg: (Gs * 1)(Gs(*seg))
    assert L.tb_ternary_gemv_multi(one(A, 1, B, C, 128, 1024, D, 1, 3), 1, s) == 2       # parts not 1, 2, 4, 8
    assert L.tb_ternary_gemv_multi(one(A, 1, B, C, 128, 1024, D, 1, 16), 1, s) == 2
    assert L.tb_ternary_gemv_multi(one(A, 1, B, C, 128, 384, D, 1, 4), 1, s) == 2        # 3 groups < 4 parts
    assert L.tb_ternary_gemv_multi(one(A, 2, B, C, 128, 384, D, 1, 4), 1, s) == 2        # any batch: G >= parts
    assert L.tb_ternary_gemv_multi(one(A, 0, B, C, 128, 1024, D, 1, 2), 1, s) == 0       # empty batch: no-op
    # two parts of [1][128] fp32 span 1 KB: a second y 512 bytes on overlaps them
    two = (Gs * 2)(Gs(A, 1, B, C, 128, 1024, D, 1, 2), Gs(A, 1, B, C, 128, 1024, D + 512, 1, 1))
    assert L.tb_ternary_gemv_multi(two, 2, s) == 8
    ok = (Gs * 2)(Gs(A, 1, B, C, 128, 1024, D, 1, 2), Gs(A, 1, B, C, 128, 1024, D + 1024, 1, 1))
    assert L.tb_ternary_gemv_multi(ok, 0, s) == 0
    # tb_fwht_segment.x_parts: fp32 partial inputs summed before the transform
    f32 = lambda x, y, rows, k, parts, res=0: F(x, y, rows, k, tb.TB_F32, tb.TB_F32, parts, res)
    assert L.tb_fwht128_multi((F * 1)(F(A, B, 1, 128, tb.TB_BF16, tb.TB_F32, 2, 0)), 1, s) == 4  # bf16 parts
    assert L.tb_fwht128_multi((F * 1)(f32(A, B, 1, 128, 9)), 1, s) == 2              # more than TB_MAX_PARTS
    assert L.tb_fwht128_multi((F * 1)(f32(A, B, 1, 128, -1)), 1, s) == 2
    assert L.tb_fwht128_multi((F * 1)(f32(A, B, 1, 128, 2, 1)), 1, s) == 2           # reserved must be 0
    assert L.tb_fwht128_multi((F * 1)(f32(A, A, 1, 128, 2)), 1, s) == 8              # in place over parts
    # four parts of one fp32 row (2 KB): an output 1.5 KB on overlaps the last part
    assert L.tb_fwht128_multi((F * 1)(f32(A, A + 1536, 1, 128, 4)), 1, s) == 8
    # another segment reading where this one's parts lie
    clash = (F * 2)(f32(A, B, 1, 128, 4), F(C, A + 1536, 1, 128, tb.TB_F32, tb.TB_F32, 1, 0))
    assert L.tb_fwht128_multi(clash, 2, s) == 8


def test_gemm_validation():
    L = tb.lib()
    s = None
    assert L.tb_ternary_gemm(_v(A), 4, _v(B), _v(C), 128, 128, _v(D), 9, s) == 4   # bad dtype
    assert L.tb_ternary_gemm(_v(A), -4, _v(B), _v(C), 128, 128, _v(D), 1, s) == 2
    assert L.tb_ternary_gemm(_v(A), 4, _v(B), _v(C), 128, 200, _v(D), 1, s) == 2
    assert L.tb_ternary_gemm(_v(A), 4, _v(B), None, 128, 128, _v(D), 1, s) == 1
    assert L.tb_ternary_gemm(_v(MIS), 4, _v(B), _v(C), 128, 128, _v(D), 1, s) == 3
    assert L.tb_ternary_gemm(_v(A), 4, _v(B), _v(C), 128, 128, _v(A), 0, s) == 8
    assert L.tb_ternary_gemm(None, 0, None, None, 128, 128, None, 1, s) == 0
    kmax = 1 << 24                                                                  # TB_GEMM_MAX_K
    assert L.tb_ternary_gemm(_v(A), 4, _v(B), _v(C), 128, kmax + 128, _v(D), 1, s) == 2
    assert L.tb_ternary_gemm_splitk(_v(A), 4, _v(B), _v(C), 128, kmax + 128, _v(D), 1, None, 0, s) == 2
    assert L.tb_ternary_gemm_rotated(_v(A), 4, _v(B), _v(C), 128, kmax + 128, _v(D), 1, None, 0, s) == 2
    assert tb.tb_ternary_gemm_splitk_workspace(16, 5120, kmax + 128) == 0
    assert tb.tb_ternary_gemm_splitk_workspace(16, 5120, kmax) > 0                  # the limit itself is taken
    S = tb.GemmSegment
    long_k = (S * 1)(S(A, B, C, 0x60000, 16, 128, kmax + 128, tb.TB_F32, 0))
    assert L.tb_ternary_gemm_multi(long_k, 1, s) == 2


def test_gemm_splitk_validation_and_workspace_size():
    L = tb.lib()
    s = None
    # the split count of the time model: 20 tiles of 64 x 256 for M = 64, N =
    # 5120 take 8 splits of K = 5120 (5 groups each) and 12 of K = 17408
    assert tb.tb_ternary_gemm_splitk_workspace(64, 5120, 5120) == 8 * 64 * 5120 * 4
    assert tb.tb_ternary_gemm_splitk_workspace(16, 5120, 17408) == 12 * 16 * 5120 * 4
    assert tb.tb_ternary_gemm_splitk_workspace(2048, 17408, 5120) == 0                 # enough tiles already
    assert tb.tb_ternary_gemm_splitk_workspace(16, 128, 256) == 0                      # too little work to split
    for m, n, k in ((1, 128, 256), (17, 256, 640), (32, 5120, 17408), (256, 17408, 5120), (64, 128, 1024)):
        ws = tb.tb_ternary_gemm_splitk_workspace(m, n, k)
        assert ws % (m * n * 4) == 0 and ws // (m * n * 4) <= min(16, k // 128)    # at most one split per group
    assert tb.tb_ternary_gemm_splitk_workspace(0, 128, 128) == 0
    assert tb.tb_ternary_gemm_splitk_workspace(16, 100, 128) == 0
    ws = 0x50000
    assert L.tb_ternary_gemm_splitk(_v(A), 4, _v(B), _v(C), 128, 128, _v(D), 9, _v(ws), 4096, s) == 4
    assert L.tb_ternary_gemm_splitk(_v(A), 4, _v(B), _v(C), 128, 200, _v(D), 1, _v(ws), 4096, s) == 2
    assert L.tb_ternary_gemm_splitk(_v(A), 4, None, _v(C), 128, 128, _v(D), 1, _v(ws), 4096, s) == 1
    assert L.tb_ternary_gemm_splitk(_v(A), 4, _v(B), _v(C), 128, 128, _v(D), 1, _v(MIS), 4096, s) == 3
    assert L.tb_ternary_gemm_splitk(_v(A), 4, _v(B), _v(C), 128, 128, _v(D), 1, _v(D + 16), 4096, s) == 8  # ws over y
    assert L.tb_ternary_gemm_splitk(_v(A), 4, _v(B), _v(C), 128, 128, _v(D), 1, _v(B + 16), 4096, s) == 8  # ws over codes
    assert L.tb_ternary_gemm_splitk(None, 0, None, None, 128, 128, None, 1, None, 0, s) == 0


def test_gemm_rotated_validation():
    L = tb.lib()
    s = None
    assert L.tb_ternary_gemm_rotated(_v(A), 4, _v(B), _v(C), 128, 128, _v(D), 9, None, 0, s) == 4
    assert L.tb_ternary_gemm_rotated(_v(A), 4, _v(B), _v(C), 100, 128, _v(D), 1, None, 0, s) == 2
    assert L.tb_ternary_gemm_rotated(_v(A), 4, _v(B), None, 128, 128, _v(D), 1, None, 0, s) == 1
    assert L.tb_ternary_gemm_rotated(_v(A), 4, _v(B), _v(C), 128, 128, _v(MIS), 1, None, 0, s) == 3
    assert L.tb_ternary_gemm_rotated(_v(A), 4, _v(B), _v(C), 128, 128, _v(A), 0, None, 0, s) == 8    # y over x
    assert L.tb_ternary_gemm_rotated(_v(A), 4, _v(B), _v(C), 128, 128, _v(D), 1, _v(C), 4096, s) == 8  # ws over scales
    assert L.tb_ternary_gemm_rotated(None, 0, None, None, 128, 128, None, 1, None, 0, s) == 0


def test_binding_raises_typed_error_on_cpu_tensors():
    import torch

    with pytest.raises(ValueError):
        tb.tb_fwht128(torch.zeros(1, 128, dtype=torch.bfloat16))


def test_binding_checks_the_act8_operand_size():
    import torch

    ok = torch.zeros(tb.tb_act8_bytes(3, 256), dtype=torch.uint8)
    tb._act8_operand(ok, 3, 256, "t")
    tb._act8_operand(ok, 0, 256, "t")  # an empty batch reads nothing
    for bad, batch in ((ok, 2), (ok[:-1], 3), (ok.view(torch.int32), 3), (torch.zeros(0, dtype=torch.uint8), 1)):
        with pytest.raises(ValueError):
            tb._act8_operand(bad, batch, 256, "t")
    with pytest.raises(ValueError):
        tb._act8_operand(ok, None, 256, "t")
