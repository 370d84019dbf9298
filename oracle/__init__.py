"""CPU oracle for C = A * B (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never loads it, and it
never loads the HIP library: the two share no code.

The arithmetic lives in ``oracle_gemm.c`` (plain C, exact decoding of every
input to double, sequential double accumulation in increasing k; int8 in
int64 reduced modulo 2^32).  This package only compiles that file with gcc
and marshals numpy arrays into it.
"""
from .oracle import (  # noqa: F401
    DTYPES, LAYOUTS, SRC, OracleLib, build, default, lib_path, gemm, gemm_entries,
    f16_bits_to_double, bf16_bits_to_double, num_threads,
)
