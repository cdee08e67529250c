"""Fused chunked top-K KL distillation loss for AMD MI355X (gfx950).

The compute path is the HIP library ``libkdchunk.so`` behind a C ABI
(``include/kd_chunked.h``); the Python binding in this package only marshals
arguments to it.
"""
