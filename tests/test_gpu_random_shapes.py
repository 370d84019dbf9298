"""Seeded random configurations against the oracle: M, N and K (ragged, and
for the register-staged variant unaligned), dtype, layout, tile class,
stages, variant, padded leading dimensions, element-aligned pointers and
split counts, drawn together so that combinations the structured tests do
not enumerate are exercised.  Each case prints its parameters first.
"""
import random

import pytest
import torch

from software_pipelined_tiled_02_amd import binding, inputs
from tests.gpu_util import EPC, alloc_c, check_close, check_sentinel, oracle_full, place

pytestmark = pytest.mark.gpu

DTYPES = ("i8", "f16", "bf16", "f32")
TILES = ("auto", "256x256", "256x256w8", "128x128", "32x64")
DIST = {"i8": "int", "f16": "normal", "bf16": "uniform", "f32": "uniform"}


def draw(rng):
    dtype = rng.choice(DTYPES)
    layout = rng.choice(("RR", "RC"))
    variant = rng.choice(("reg", "direct"))
    e = EPC[dtype]
    M = rng.randint(1, 700)
    N = rng.randint(1, 600)
    K = rng.randint(1, 3000)
    if layout == "RR":
        N = max(e, N // e * e)                      # layout RR: N in whole 16-byte chunks
    pad, off = 0, 0
    if variant == "direct":
        K = max(e, K // e * e)
        pad = e * rng.randint(0, 2)
    else:
        pad, off = rng.randint(0, 5), rng.randint(0, 3)
    return dict(dtype=dtype, layout=layout, variant=variant, stages=rng.randint(1, 4),
                tile=rng.choice(TILES), splits=rng.choice((1, 1, 2, 3, 5)), M=M, N=N, K=K, pad=pad, off=off)


CASES = [draw(random.Random(1000 + i)) for i in range(48)]
# The 3-stage direct ring of the 256x256 tiles (split by operand): more
# cases of it than the draw above gives, with every other option random and
# K long enough for the ring to wrap several times.
SPLIT_RING = []
for i in range(16):
    rng = random.Random(5000 + i)
    case = draw(rng)
    e = EPC[case["dtype"]]
    K = max(e, rng.randint(300, 4000) // e * e)
    case.update(variant="direct", stages=3, tile=rng.choice(("256x256", "256x256w8")), K=K,
                pad=e * rng.randint(0, 2), off=0, M=rng.randint(200, 700), N=case["N"] if case["layout"] == "RR"
                else rng.randint(200, 600))
    SPLIT_RING.append(case)
CASES += SPLIT_RING


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gg = binding.Gemm(0)
    yield gg
    gg.close()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%(dtype)s-%(layout)s-%(variant)s-S%(stages)d-%(tile)s-"
                                                      "p%(splits)d-%(M)dx%(N)dx%(K)d" % c)
def test_random_case(g, case):
    print("case:", case, flush=True)
    dtype, layout, M, N, K = case["dtype"], case["layout"], case["M"], case["N"], case["K"]
    a, b = inputs.make_operands(M, N, K, dtype, layout, DIST[dtype], seed=M * 7 + N * 3 + K)
    ref = oracle_full(a, b, dtype, layout)
    lda = K + case["pad"]
    ldb = (N if layout == "RR" else K) + case["pad"]
    ldc = (N + 3) // 4 * 4
    a_buf, a_ptr = place(a, lda, case["off"], dtype)
    b_buf, b_ptr = place(b, ldb, case["off"], dtype)
    c = alloc_c(M, N, ldc, dtype)
    g.set_tile(case["tile"])
    try:
        _, info = binding.gemm_query(M, N, K, dtype, layout, case["stages"], case["variant"], tile=case["tile"],
                                     lda=lda, ldb=ldb, ldc=ldc, splits=case["splits"])
        ws = g.workspace(info["workspace_bytes"]) if info["workspace_bytes"] else None
        binding.gemm_run_splitk(g.h, M, N, K, dtype, layout, case["stages"], case["variant"], case["splits"],
                                a_ptr, lda, b_ptr, ldb, c, ldc, ws, ws.numel() if ws is not None else 0)
        torch.cuda.synchronize()
    finally:
        g.set_tile("auto")
    c = c.cpu()
    check_sentinel(c, M, N, dtype)
    check_close(c[:M, :N], ref, dtype, str(case))
    del a_buf, b_buf
