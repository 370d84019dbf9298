"""ctypes front end of the C oracle (test infrastructure only).

Matrices are numpy arrays in the oracle's own element encodings:
  int8  -> numpy.int8
  fp16  -> numpy.uint16 holding IEEE binary16 bit patterns
  bf16  -> numpy.uint16 holding bfloat16 bit patterns
  fp32  -> numpy.float32
A is row-major M x K.  B is row-major K x N for layout "RR" and column-major
(stored as an N x K row-major array, K contiguous) for layout "RC".
The result is int32 for int8 inputs and float64 otherwise.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle_gemm.so")

DTYPES = {"i8": 0, "f16": 1, "bf16": 2, "f32": 3}
LAYOUTS = {"RR": 0, "RC": 1}
_NP_IN = {"i8": np.int8, "f16": np.uint16, "bf16": np.uint16, "f32": np.float32}


def lib_path():
    return _LIB


def build(src=SRC, out=None):
    """Compile an oracle source file with gcc into a shared library."""
    out = out or _LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class OracleLib:
    """One loaded copy of the oracle library."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_gemm.argtypes = [ci, ci, i64, i64, i64, vp, i64, vp, i64, vp, i64]
        lib.oracle_gemm.restype = ci
        lib.oracle_gemm_entries.argtypes = [ci, ci, i64, i64, i64, vp, i64, vp, i64,
                                            i64, vp, vp, vp]
        lib.oracle_gemm_entries.restype = ci
        lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_num_threads.restype = ci
        self.lib = lib
        self.path = path

    @staticmethod
    def _check(a, b, dtype, layout):
        if dtype not in DTYPES or layout not in LAYOUTS:
            raise ValueError("bad dtype/layout %r/%r" % (dtype, layout))
        want = _NP_IN[dtype]
        if a.dtype != want or b.dtype != want:
            raise TypeError("oracle %s expects %s arrays" % (dtype, np.dtype(want)))
        if a.ndim != 2 or b.ndim != 2:
            raise ValueError("A and B must be 2-D")
        for x in (a, b):
            if x.size and x.shape[1] > 1 and x.strides[1] != x.itemsize:
                raise ValueError("A and B need a unit stride along their last axis")
            if x.size and x.shape[0] > 1 and (x.strides[0] % x.itemsize
                                              or x.strides[0] // x.itemsize < x.shape[1]):
                raise ValueError("rows of A and B must not overlap")
        M, K = a.shape
        if layout == "RR":
            K2, N = b.shape
        else:
            N, K2 = b.shape
        if K2 != K:
            raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
        return M, N, K

    @staticmethod
    def _ld(x):
        if x.size == 0 or x.shape[0] == 1:
            return max(x.shape[1], 1)
        return x.strides[0] // x.itemsize

    def gemm(self, a, b, dtype, layout):
        """Full C = A * B; int32 for int8 inputs, float64 otherwise."""
        M, N, K = self._check(a, b, dtype, layout)
        out = np.zeros((M, N), dtype=np.int32 if dtype == "i8" else np.float64)
        rc = self.lib.oracle_gemm(DTYPES[dtype], LAYOUTS[layout], M, N, K,
                                  a.ctypes.data, self._ld(a), b.ctypes.data, self._ld(b),
                                  out.ctypes.data, max(N, 1))
        if rc != 0:
            raise ValueError("oracle_gemm rejected its arguments")
        return out

    def gemm_entries(self, a, b, dtype, layout, rows, cols):
        """C(rows[t], cols[t]) for each t, in the same arithmetic as gemm()."""
        M, N, K = self._check(a, b, dtype, layout)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape or rows.ndim != 1:
            raise ValueError("rows and cols must be 1-D and equally long")
        out = np.zeros(rows.shape, dtype=np.int32 if dtype == "i8" else np.float64)
        rc = self.lib.oracle_gemm_entries(DTYPES[dtype], LAYOUTS[layout], M, N, K,
                                          a.ctypes.data, self._ld(a), b.ctypes.data,
                                          self._ld(b), rows.size, rows.ctypes.data,
                                          cols.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_gemm_entries rejected its arguments")
        return out

    def f16_bits_to_double(self, bits):
        return self.lib.oracle_f16_to_double(int(bits))

    def bf16_bits_to_double(self, bits):
        return self.lib.oracle_bf16_to_double(int(bits))

    def num_threads(self):
        return self.lib.oracle_num_threads()


_default = None


def default():
    """The oracle built from oracle_gemm.c (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = OracleLib(_LIB)
    return _default


def gemm(a, b, dtype, layout):
    return default().gemm(a, b, dtype, layout)


def gemm_entries(a, b, dtype, layout, rows, cols):
    return default().gemm_entries(a, b, dtype, layout, rows, cols)


def f16_bits_to_double(bits):
    return default().f16_bits_to_double(bits)


def bf16_bits_to_double(bits):
    return default().bf16_bits_to_double(bits)


def num_threads():
    return default().num_threads()
