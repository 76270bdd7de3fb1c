"""CPU oracle for inference with Hadamard-rotated ternary weights.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It is plain numpy float64 code,
deliberately slow and obvious, and it shares no code, tables or helpers with
the HIP library under ``ternary_weights_hadamard_amd/``.

The reference material is a set of web pages with no titles of their own in
the extracted text; they are cited by address and by the page's own section
numbers:

* dpshk.com/news/5289456  - TensorSharp walkthrough (bit-rule Hadamard, 128x128
  blocks, "divide by 128", sign/magnitude storage, conversion steps).
* xxqk.cn/news/652513     - H.W.H^T and the butterfly transform, A100 timings.
* mhpq.cn/news/1159370    - absmean ternarisation, 2:4 pruning, per-128 fp16
  scale, the 1.585 + 0.125 bit ledger, 2-bit packing.
* zwxr.cn/news/303439     - Hadamard identities y = Hx, x = (1/n) H y.

Modules
-------
``numerics``  fp16 / bf16 round-to-nearest-even by integer bit operations.
``hadamard``  H by the bit rule and by Sylvester's recursion; blockwise FWHT128
              (dense matmul and butterfly forms); the 2D block rotation.
``quant``     absmean group scale, ternarisation, dense and 2:4 packing; the
              error-minimising threshold rule; the residual second plane.
``matvec``    the ternary GEMV / GEMM / 2:4 GEMV / two-plane GEMV definitions
              (dequantise, then a float64 matmul) and brute-force loop versions.
``bits``      bits-per-weight ledger and packed buffer sizes.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library routines or brute force; none is "parity
unpinned".
"""

from . import bits, hadamard, matvec, numerics, quant  # noqa: F401
