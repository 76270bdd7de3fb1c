"""tb_ternary_gemv_noalloc (the GEMV for callers that cannot allocate) against
tb_ternary_gemv with bf16 activations and a caller workspace: bit-equal on two
calls in a row, the second with a smaller input, called through the C ABI."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, assert_close, bf16_dev, f16_dev, say, u32_dev
from ternary_weights_hadamard_amd import synth, tb

pytestmark = pytest.mark.gpu


def _noalloc(x, cd, sc, y):
    L = tb.lib()
    n, g = sc.shape[0] * 16, sc.shape[1]
    st = L.tb_ternary_gemv_noalloc(ctypes.c_void_p(x.data_ptr()), x.shape[0], ctypes.c_void_p(cd.data_ptr()),
                                   ctypes.c_void_p(sc.data_ptr()), n, g * 128, ctypes.c_void_p(y.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, tb.status_string(st)


def _with_workspace(x, cd, sc):
    b, k = x.shape
    ws = torch.empty(tb.tb_act8_bytes(b, k), dtype=torch.uint8, device=DEV)
    return tb.tb_ternary_gemv(x, cd, sc, workspace=ws)


def test_noalloc_equals_the_workspace_entry_on_two_calls_in_a_row():
    # first call: batch 16, a 27B down projection's K (the scratch's largest use
    # here); second: a smaller batch and K, so stale bytes of the first call sit
    # in the scratch past what the second one writes
    for n, k, b, seed in ((1024, 17408, 16, 501), (384, 1152, 3, 502)):
        say(f"no-alloc gemv N={n} K={k} B={b}")
        codes = synth.random_code_words(n, k, seed=seed)
        scales = synth.random_scales_f16(n, k, seed=seed + 1)
        x = synth.gaussian_bf16((b, k), seed=seed + 2)
        xd, cd, sc = bf16_dev(x), u32_dev(codes), f16_dev(scales)
        y = torch.full((b, n), 7.0, dtype=torch.float32, device=DEV)
        _noalloc(xd, cd, sc, y)
        ref_ws = _with_workspace(xd, cd, sc)
        torch.cuda.synchronize()
        assert torch.equal(y, ref_ws), f"no-alloc differs from the workspace entry at N={n} K={k} B={b}"
        assert_close(y.cpu().numpy(), oracle.matvec.gemv(x, codes, scales, k), f"no-alloc {n}x{k} B={b}")


def test_noalloc_rejects_an_input_beyond_its_scratch():
    L = tb.lib()
    big_k = 63488 + 128  # tb_act8_bytes(16, K) exceeds 4 MiB
    assert tb.tb_act8_bytes(16, big_k) > tb.TB_NOALLOC_SCRATCH_BYTES >= tb.tb_act8_bytes(16, 63488)
    a = ctypes.c_void_p(0x10000)
    assert L.tb_ternary_gemv_noalloc(a, 16, ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x30000000), 128, big_k,
                                     ctypes.c_void_p(0x40000000), None) == 9
