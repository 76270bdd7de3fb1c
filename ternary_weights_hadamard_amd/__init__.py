"""Hadamard-rotated ternary weights on MI355X (gfx950).

The compute path is the C-ABI library ``libtb.so`` built from ``csrc/``; the
``tb`` module is a thin ctypes binding over it.  Import ``synth`` for seeded
inputs.  Nothing here falls back to a CPU implementation: when the library is
missing every call raises.
"""
