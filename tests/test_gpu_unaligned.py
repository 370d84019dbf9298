"""GPU parity for K and leading dimensions that are not whole 16-byte chunks
and for operand pointers that are only element-aligned: the register-staged
variant, every tile class and pipeline depth, against the oracle.

The K loop is the one the tiled GEMM's pipelining restructures ("CUDA Kernel
Study: Pipelining", Example Code); the fallback for a last tile that cannot
be copied in whole aligned pieces -- smaller bounds-checked loads -- is the
one the skill names ("pipeline-gpu-kernel", pitfalls, cp.async boundary
handling).
Operands sit in buffers that end at their last element, with NaN (int8:
0x55) in the row padding and before the first element, so a read of any
byte past K shows up in C.  The direct-to-LDS variant moves whole 16-byte
chunks and must refuse these calls.
"""
import pytest
import torch

from software_pipelined_tiled_02_amd import binding, inputs
from tests.gpu_util import EPC, check_close, check_sentinel, oracle_full, run_gpu_placed

pytestmark = pytest.mark.gpu

DTYPES = ("i8", "f16", "bf16", "f32")
STAGES = (1, 2, 3, 4)
LAYOUT_TILES = [("RC", "256x256"), ("RC", "256x256w8"), ("RC", "128x128"), ("RC", "32x64"),
                ("RR", "256x256"), ("RR", "256x256w8"), ("RR", "128x128"), ("RR", "32x64")]
DIST = {"i8": "int", "f16": "normal", "bf16": "uniform", "f32": "uniform"}
# K below one chunk, a little over one, several K-tiles with a ragged chunk,
# and a whole number of chunks (then only the rows are unaligned)
KS = {"i8": (3, 17, 1001, 128), "f16": (5, 9, 1001, 64), "bf16": (1, 13, 1001, 64),
      "f32": (3, 5, 999, 32)}
# (extra elements per row, pointer offset in elements)
ROWS = ((0, 1), (1, 0), (3, 3))


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gg = binding.Gemm(0)
    yield gg
    gg.close()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout,tile", LAYOUT_TILES)
def test_unaligned_k_and_rows(g, dtype, layout, tile):
    """Every depth matches the oracle and, per (K, rows), the others bit for bit."""
    M, N = 130, 80
    g.set_tile(tile)
    try:
        for K in KS[dtype]:
            a, b = inputs.make_operands(M, N, K, dtype, layout, DIST[dtype], seed=K)
            ref = oracle_full(a, b, dtype, layout)
            for pad, off in ROWS:
                lda = K + pad
                ldb = (N if layout == "RR" else K) + pad
                first = None
                for stages in STAGES:
                    what = "%s %s %s K=%d lda=%d ldb=%d off=%d S=%d reg" % (
                        dtype, layout, tile, K, lda, ldb, off, stages)
                    print("case:", what, flush=True)
                    _, c = run_gpu_placed(g, a, b, dtype, layout, stages, "reg", M, N, K, lda, ldb, off)
                    check_sentinel(c, M, N, dtype)
                    check_close(c[:M, :N], ref, dtype, what)
                    if first is None:
                        first = c
                    else:
                        assert torch.equal(c.view(torch.uint8), first.view(torch.uint8)), \
                            what + ": not bit-identical to S=1"
    finally:
        g.set_tile("auto")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", ("RR", "RC"))
def test_unaligned_larger(g, dtype, layout):
    """Many tiles in M and N and a long K with a ragged chunk, auto tile."""
    M, N, K = 600, 528, 4096 + EPC[dtype] // 2 + 1
    a, b = inputs.make_operands(M, N, K, dtype, layout, DIST[dtype], seed=7)
    ref = oracle_full(a, b, dtype, layout)
    for stages in (2, 3):
        what = "%s %s K=%d S=%d reg" % (dtype, layout, K, stages)
        print("case:", what, flush=True)
        _, c = run_gpu_placed(g, a, b, dtype, layout, stages, "reg", M, N, K, K + 1,
                              (N if layout == "RR" else K) + 1, 1)
        check_sentinel(c, M, N, dtype)
        check_close(c[:M, :N], ref, dtype, what)


@pytest.mark.parametrize("dtype", DTYPES)
def test_direct_refuses_unaligned(g, dtype):
    """The direct variant returns GEMM_ERR_ALIGNMENT and leaves C alone."""
    M, N, K = 64, 64, 3 * EPC[dtype] + 1
    a, b = inputs.make_operands(M, N, K, dtype, "RC", DIST[dtype], seed=1)
    for K_, lda, off in ((K, K, 0), (K - 1, K, 0), (K - 1, K - 1, 1)):
        rc, c = run_gpu_placed(g, a[:, :K_].contiguous(), b[:, :K_].contiguous(), dtype, "RC", 2,
                               "direct", M, N, K_, lda, lda, off, check=False)
        assert rc == binding.GEMM_ERR_ALIGNMENT, (dtype, K_, lda, off, rc)
        check_sentinel(c, 0, N, dtype)
