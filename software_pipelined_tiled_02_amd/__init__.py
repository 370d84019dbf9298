"""pipegemm: a software-pipelined tiled GEMM for AMD Instinct MI355X (gfx950).

The kernels live in ``csrc/`` (hand-written HIP) behind the C ABI declared in
``include/pipegemm.h``; ``binding`` is the thin ctypes layer over it.  Import
of this package loads nothing: the library is opened on first use.
"""
