"""kvq: quantized KV-cache rows and decode attention, native on MI355X (gfx950).

The compute path is the C-ABI library libkvq.so (hand-written HIP kernels);
this package is a thin ctypes binding over it (see ``kvq.py``).
"""
