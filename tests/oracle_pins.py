"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes an ``oracle.OracleLib`` and raises
AssertionError when that library disagrees with what the mathematics or the
pages fix:
  - hand-worked products of the plain definition (tests/golden),
  - an independent library routine (numpy matmul in int64/float64; numpy's
    and torch's own fp16/bf16 decoders),
  - exact brute force in Python integers / fractions on tiny shapes,
  - closed forms: identity and permutation operands, all-ones (C == K),
    row sums against a separate 1-D loop,
  - the int32 wrap-around of the integer reference.
The same functions run against deliberately broken copies of the oracle in
test_oracle.py, which must each fail at least one pin.
"""
import json
import os
from fractions import Fraction

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "matmul_worked_examples.json")

FLOAT_DTYPES = ("f16", "bf16", "f32")
ALL_DTYPES = ("i8",) + FLOAT_DTYPES
LAYOUTS = ("RR", "RC")


# ---- encoders used only to build test operands --------------------------

def encode(values, dtype):
    """float/int numpy array -> the oracle's storage for dtype."""
    v = np.asarray(values)
    if dtype == "i8":
        return v.astype(np.int8)
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    t = torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def decode_lib(x, dtype):
    """Oracle storage -> float64 (or int64) via numpy/torch's own decoders."""
    if dtype == "i8":
        return x.astype(np.int64)
    if dtype == "f32":
        return x.astype(np.float64)
    if dtype == "f16":
        return x.view(np.float16).astype(np.float64)
    t = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16)
    return t.double().numpy()


def b_storage(b_kxn, layout):
    """A K x N matrix in the layout's storage (RC stores its N x K transpose)."""
    return np.ascontiguousarray(b_kxn if layout == "RR" else b_kxn.T)


def padded(x, extra):
    """Same matrix with a leading dimension larger than its row length."""
    if extra == 0:
        return np.ascontiguousarray(x)
    big = np.zeros((x.shape[0], x.shape[1] + extra), dtype=x.dtype)
    big[:, : x.shape[1]] = x
    return big[:, : x.shape[1]]


def random_values(rng, shape, dtype):
    if dtype == "i8":
        return rng.integers(-128, 128, size=shape)
    return rng.standard_normal(shape)


def _exact_decoded(x, dtype):
    d = decode_lib(x, dtype)
    if dtype == "i8":
        return [[int(v) for v in row] for row in d]
    return [[Fraction(float(v)) for v in row] for row in d]


# ---- pins -----------------------------------------------------------------

def pin_golden(orc):
    g = json.load(open(GOLDEN))
    for ex in g["examples"]:
        a = np.array(ex["A"])
        b = np.array(ex["B_KxN"])
        want = np.array(ex["C"])
        for dtype in ALL_DTYPES:
            for layout in LAYOUTS:
                c = orc.gemm(encode(a, dtype), b_storage(encode(b, dtype), layout), dtype, layout)
                assert np.array_equal(c, want), (ex["name"], dtype, layout, c)
    w = g["int8_wrap"]
    a = np.full((1, w["K"]), w["a_value"], dtype=np.int8)
    bt = np.full((1, w["K"]), w["b_value"], dtype=np.int8)
    c = orc.gemm(a, bt, "i8", "RC")
    assert int(c[0, 0]) == w["wrapped_int32"], c
    c = orc.gemm(a, np.ascontiguousarray(bt.T), "i8", "RR")
    assert int(c[0, 0]) == w["wrapped_int32"], c


def pin_decoders(orc):
    """Every one of the 65536 fp16 and bf16 bit patterns decodes as numpy /
    torch decode it (NaN patterns to a NaN)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref16 = bits.view(np.float16).astype(np.float64)
    refbf = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    for i in range(65536):
        got = orc.f16_bits_to_double(i)
        if np.isnan(ref16[i]):
            assert np.isnan(got), i
        else:
            assert got == ref16[i], (hex(i), got, ref16[i])
        got = orc.bf16_bits_to_double(i)
        if np.isnan(refbf[i]):
            assert np.isnan(got), i
        else:
            assert got == refbf[i], (hex(i), got, refbf[i])


def pin_brute_force(orc):
    """Tiny shapes against exact Python-integer / rational arithmetic.

    int8 must match exactly.  Floats must lie within the error bound of a
    sequential double sum: |s - exact| <= K * 2^-53 * sum_k |a_ik b_kj|.
    """
    rng = np.random.default_rng(1234)
    shapes = [(1, 1, 1), (2, 3, 5), (3, 2, 1), (5, 7, 8), (8, 8, 3), (4, 1, 7), (1, 6, 4)]
    for dtype in ALL_DTYPES:
        for layout in LAYOUTS:
            for (M, N, K) in shapes:
                a = encode(random_values(rng, (M, K), dtype), dtype)
                b = encode(random_values(rng, (K, N), dtype), dtype)
                extra = (M + N + K) % 3
                c = orc.gemm(padded(a, extra), padded(b_storage(b, layout), extra), dtype, layout)
                ea, eb = _exact_decoded(a, dtype), _exact_decoded(b, dtype)
                for i in range(M):
                    for j in range(N):
                        terms = [ea[i][k] * eb[k][j] for k in range(K)]
                        exact = sum(terms, 0 if dtype == "i8" else Fraction(0))
                        if dtype == "i8":
                            assert int(c[i, j]) == exact, (dtype, layout, M, N, K, i, j)
                        else:
                            bound = K * 2.0 ** -53 * float(sum(abs(t) for t in terms))
                            assert abs(Fraction(float(c[i, j])) - exact) <= Fraction(bound), \
                                (dtype, layout, M, N, K, i, j, c[i, j], float(exact))


def pin_numpy_matmul(orc):
    """Medium shapes against numpy matmul on the independently decoded inputs."""
    rng = np.random.default_rng(99)
    for dtype in ALL_DTYPES:
        for layout in LAYOUTS:
            for (M, N, K) in [(33, 17, 64), (64, 48, 129), (7, 70, 300)]:
                a = encode(random_values(rng, (M, K), dtype), dtype)
                b = encode(random_values(rng, (K, N), dtype), dtype)
                c = orc.gemm(a, b_storage(b, layout), dtype, layout)
                ref = decode_lib(a, dtype) @ decode_lib(b, dtype)
                if dtype == "i8":
                    assert np.array_equal(c.astype(np.int64), ref), (dtype, layout, M, N, K)
                else:
                    scale = np.abs(decode_lib(a, dtype)) @ np.abs(decode_lib(b, dtype))
                    assert np.all(np.abs(c - ref) <= 4 * K * 2.0 ** -53 * scale + 1e-300), \
                        (dtype, layout, M, N, K, np.max(np.abs(c - ref)))


def pin_identity_and_permutation(orc):
    """A = I gives C = B and A = P gives the rows of B permuted, bit-exactly;
    B = P (K = N) gives the columns of A permuted."""
    rng = np.random.default_rng(7)
    for dtype in ALL_DTYPES:
        for layout in LAYOUTS:
            K, N, M = 24, 19, 24
            b = encode(random_values(rng, (K, N), dtype), dtype)
            bd = decode_lib(b, dtype)
            eye = encode(np.eye(M, K), dtype)
            c = orc.gemm(eye, b_storage(b, layout), dtype, layout)
            assert np.array_equal(c, bd), (dtype, layout, "identity")
            perm = rng.permutation(K)
            p = np.zeros((M, K))
            p[np.arange(M), perm] = 1
            c = orc.gemm(encode(p, dtype), b_storage(b, layout), dtype, layout)
            assert np.array_equal(c, bd[perm, :]), (dtype, layout, "row permutation")
            # B = permutation with N = K: C[:, j] = A[:, q(j)]
            Mx, Kx = 11, 16
            a = encode(random_values(rng, (Mx, Kx), dtype), dtype)
            q = rng.permutation(Kx)
            pb = np.zeros((Kx, Kx))
            pb[q, np.arange(Kx)] = 1
            c = orc.gemm(a, b_storage(encode(pb, dtype), layout), dtype, layout)
            assert np.array_equal(c, decode_lib(a, dtype)[:, q]), (dtype, layout, "column permutation")


def pin_all_ones_and_row_sums(orc):
    """A = B = 1 gives C == K exactly; B = 1 gives C_ij = sum_k A_ik."""
    rng = np.random.default_rng(5)
    for dtype in ALL_DTYPES:
        for layout in LAYOUTS:
            for (M, N, K) in [(3, 5, 1), (9, 4, 37), (16, 16, 1000)]:
                ones_a = encode(np.ones((M, K)), dtype)
                ones_b = encode(np.ones((K, N)), dtype)
                c = orc.gemm(ones_a, b_storage(ones_b, layout), dtype, layout)
                assert np.all(c == K), (dtype, layout, M, N, K)
                a = encode(random_values(rng, (M, K), dtype), dtype)
                c = orc.gemm(a, b_storage(ones_b, layout), dtype, layout)
                ad = decode_lib(a, dtype)
                for i in range(M):
                    if dtype == "i8":
                        rs = sum(int(v) for v in ad[i])
                        assert np.all(c[i] == rs), (dtype, layout, i)
                    else:
                        rs = sum((Fraction(float(v)) for v in ad[i]), Fraction(0))
                        bound = K * 2.0 ** -53 * float(np.sum(np.abs(ad[i])))
                        for j in range(N):
                            assert abs(Fraction(float(c[i, j])) - rs) <= Fraction(bound), \
                                (dtype, layout, i, j)


def pin_entries(orc):
    """Selected entries agree with exact brute force and with the full product."""
    rng = np.random.default_rng(11)
    for dtype in ALL_DTYPES:
        for layout in LAYOUTS:
            M, N, K = 13, 9, 21
            a = encode(random_values(rng, (M, K), dtype), dtype)
            b = encode(random_values(rng, (K, N), dtype), dtype)
            rows = rng.integers(0, M, size=25)
            cols = rng.integers(0, N, size=25)
            e = orc.gemm_entries(a, b_storage(b, layout), dtype, layout, rows, cols)
            ref = decode_lib(a, dtype) @ decode_lib(b, dtype)
            for t in range(25):
                if dtype == "i8":
                    assert int(e[t]) == int(ref[rows[t], cols[t]]), (dtype, layout, t)
                else:
                    sc = float(np.abs(decode_lib(a, dtype)[rows[t]]) @ np.abs(decode_lib(b, dtype)[:, cols[t]]))
                    assert abs(e[t] - ref[rows[t], cols[t]]) <= 4 * K * 2.0 ** -53 * sc + 1e-300
            full = orc.gemm(a, b_storage(b, layout), dtype, layout)
            assert np.array_equal(e, full[rows, cols])


ALL_PINS = [pin_golden, pin_decoders, pin_brute_force, pin_numpy_matmul,
            pin_identity_and_permutation, pin_all_ones_and_row_sums, pin_entries]
