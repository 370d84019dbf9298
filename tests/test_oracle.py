"""The CPU oracle against its pins (no GPU).

Every pin in oracle_pins.py must hold for the oracle as committed, and each
planted mistake below (made in a private copy of oracle_gemm.c, compiled on
the CPU) must break at least one pin: that is what shows the pins would
catch a dropped term, a wrong sign or index, a transposed operand, a wrong
decoder or a wrong integer wrap.
"""
import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.OracleLib(oracle.lib_path())


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_arguments(orc):
    a = np.zeros((2, 3), dtype=np.float32)
    b = np.zeros((3, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        orc.gemm(a, np.zeros((2, 4), dtype=np.float32), "f32", "RR")  # K mismatch
    with pytest.raises(TypeError):
        orc.gemm(a, b.astype(np.float64), "f32", "RR")
    with pytest.raises(ValueError):
        orc.gemm(a, b, "f64", "RR")
    with pytest.raises(ValueError):
        orc.gemm_entries(a, b, "f32", "RR", [2], [0])  # row out of range


def test_oracle_empty_shapes(orc):
    for dtype, npt in (("i8", np.int8), ("f32", np.float32)):
        c = orc.gemm(np.zeros((0, 5), npt), np.zeros((5, 3), npt), dtype, "RR")
        assert c.shape == (0, 3)
        c = orc.gemm(np.zeros((4, 0), npt), np.zeros((3, 0), npt), dtype, "RC")
        assert c.shape == (4, 3) and np.all(c == 0)


# (description, text in oracle_gemm.c, replacement, occurrences expected)
MUTANTS = [
    ("dropped last k term", "k < K; ++k)", "k < K - 1; ++k)", None),
    ("B layouts swapped", "k * ldb + j : j * ldb + k", "j * ldb + k : k * ldb + j", 1),
    ("wrong sign in RC float sum", "s += arow[k] *", "s -= arow[k] *", 1),
    ("wrong fp16 exponent bias", "e - 25)", "e - 24)", 1),
    ("wrong bf16 placement", "(uint32_t)b << 16", "(uint32_t)b << 15", 1),
    ("wrong int32 wrap", "& 0xffffffffu", "& 0x7fffffffu", 1),
    ("RR row uses column of A", "load_f(dtype, A, i * lda + k);\n                    for",
     "load_f(dtype, A, i * lda + (k ? k - 1 : 0));\n                    for", 1),
    ("first term dropped in RR int loop", "acc[j] += aik * (int64_t)brow[j]",
     "acc[j] += (k ? aik : 0) * (int64_t)brow[j]", 1),
]


@pytest.mark.parametrize("desc,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(desc, old, new, count):
    src = open(oracle.SRC).read()
    n = src.count(old)
    assert n >= 1 and (count is None or n == count), (desc, n)
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        path = os.path.join(tmp, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.build(src=path, out=os.path.join(tmp, "libmutant.so"))
        mutant = oracle.OracleLib(lib)
        failed = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mutant)
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, "no pin caught: " + desc
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("layout", ["RR", "RC"])
def test_widened_inputs_give_the_same_doubles(orc, dtype, layout):
    """The full-size GPU parity tests call the oracle's fp32 entry on fp16 /
    bf16 operands widened to fp32 (exact): it must return exactly the
    doubles of the fp16 / bf16 entry.  Inputs cover subnormals, signed
    zeros, the largest finite values and ordinary values."""
    import torch
    from software_pipelined_tiled_02_amd import inputs
    rng = np.random.default_rng(7)
    M, N, K = 37, 29, 301
    tdt = inputs.TORCH_DTYPES[dtype]
    special = {"f16": [0x0001, 0x03FF, 0x8001, 0x7BFF, 0xFBFF, 0x8000, 0x0000, 0x3C00],
               "bf16": [0x0001, 0x007F, 0x8001, 0x7F7F, 0xFF7F, 0x8000, 0x0000, 0x3F80]}[dtype]

    def draw(shape):
        bits = rng.integers(0, 65536, size=shape, dtype=np.int64)
        x = torch.from_numpy(bits.astype(np.int16)).view(tdt)
        bad = ~torch.isfinite(x.float())
        x[bad] = 0.5                                   # no inf / NaN operands
        flat = x.view(-1)
        flat[: len(special)] = torch.tensor(np.array(special, dtype=np.int64).astype(np.int16)).view(tdt)
        return x.contiguous()

    a = draw((M, K))              # products and sums stay finite in double
    b = draw((K, N) if layout == "RR" else (N, K))
    ref = orc.gemm(inputs.to_oracle(a, dtype), inputs.to_oracle(b, dtype), dtype, layout)
    wid = orc.gemm(a.float().contiguous().numpy(), b.float().contiguous().numpy(), "f32", layout)
    assert np.array_equal(ref.view(np.int64), wid.view(np.int64))


_THREADS_PROBE = r"""
import sys, numpy as np
sys.path.insert(0, %r)
import oracle
orc = oracle.OracleLib(oracle.lib_path())
rng = np.random.default_rng(11)
out = [orc.num_threads()]
for dtype, layout in (("f32", "RR"), ("f32", "RC"), ("i8", "RC")):
    if dtype == "f32":
        a = rng.uniform(-1, 1, (67, 301)).astype(np.float32)
        b = rng.uniform(-1, 1, (301, 45) if layout == "RR" else (45, 301)).astype(np.float32)
    else:
        a = rng.integers(-128, 128, (67, 301)).astype(np.int8)
        b = rng.integers(-128, 128, (45, 301)).astype(np.int8)
    out.append(orc.gemm(a, b, dtype, layout).tobytes().hex())
print(repr(out))
"""


def test_oracle_threads_do_not_change_the_result(orc):
    """oracle_num_threads reports the OpenMP threads the oracle runs with
    (the core count the CPU baseline states), and the result is the same
    bits with one thread or several: each C element is one sequential sum
    in increasing k whichever thread computes it."""
    import ast
    import subprocess
    import sys
    from tests.conftest import ROOT
    got = {}
    for n in (1, 3):
        env = dict(os.environ, OMP_NUM_THREADS=str(n))
        r = subprocess.run([sys.executable, "-c", _THREADS_PROBE % ROOT], env=env, capture_output=True,
                           text=True, timeout=120, check=True)
        got[n] = ast.literal_eval(r.stdout.strip().splitlines()[-1])
        assert got[n][0] == n, (n, got[n][0])
    assert got[1][1:] == got[3][1:]
