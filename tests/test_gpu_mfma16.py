"""The 16x16 MFMA blocks on ragged shapes.

The 4-wave 256x256 tile's 2- and 3-stage direct-to-LDS instances (both
layouts) build each wave's C block from 16x16 MFMA blocks, the other
instances from 32x32 blocks.  Each seeded case here -- M and N small or ragged inside a
16-row half, K of several tiles with a ragged head, padded rows, split
counts -- asserts that the query reports 16x16 blocks for it and 32x32 for
the 1-stage instance of the same tile, checks C against the oracle, and
checks it bit for bit against that 1-stage 32x32 instance on the same
inputs.  Each case prints its parameters first.
"""
import random

import pytest
import torch

from software_pipelined_tiled_02_amd import binding, inputs
from tests.gpu_util import EPC, alloc_c, check_close, check_sentinel, oracle_full, place

pytestmark = pytest.mark.gpu

DIST = {"i8": "int", "f16": "normal", "bf16": "uniform"}


def draw(rng):
    dtype = rng.choice(("i8", "f16", "bf16"))
    e = EPC[dtype]
    small = rng.random() < 0.35
    M = rng.randint(1, 40) if small else rng.randint(200, 700)
    N = rng.randint(1, 40) if rng.random() < 0.35 else rng.randint(200, 600)
    K = max(e, rng.randint(1, 3000) // e * e)
    return dict(dtype=dtype, layout="RC", stages=rng.choice((2, 3)), splits=rng.choice((1, 1, 2, 3)), M=M, N=N,
                K=K, pad=e * rng.randint(0, 2))


def draw_rr(rng):
    case = draw(rng)
    e = EPC[case["dtype"]]
    case.update(layout="RR", N=max(e, case["N"] // e * e))   # layout RR: N in whole 16-byte chunks
    return case


CASES = [draw(random.Random(7000 + i)) for i in range(24)] + [draw_rr(random.Random(7500 + i)) for i in range(16)]


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gg = binding.Gemm(0)
    gg.set_tile("256x256")
    yield gg
    gg.set_tile("auto")
    gg.close()


def bits(t):
    t = t.contiguous()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def run(g, case, stages, a_ptr, lda, b_ptr, ldb, ldc):
    dtype, M, N, K, splits = case["dtype"], case["M"], case["N"], case["K"], case["splits"]
    layout = case["layout"]
    _, info = binding.gemm_query(M, N, K, dtype, layout, stages, "direct", tile="256x256", lda=lda, ldb=ldb,
                                 ldc=ldc, splits=splits)
    c = alloc_c(M, N, ldc, dtype)
    ws = g.workspace(info["workspace_bytes"]) if info["workspace_bytes"] else None
    binding.gemm_run_splitk(g.h, M, N, K, dtype, layout, stages, "direct", splits, a_ptr, lda, b_ptr, ldb, c, ldc,
                            ws, ws.numel() if ws is not None else 0)
    torch.cuda.synchronize()
    return info, c.cpu()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%(dtype)s-%(layout)s-S%(stages)d-p%(splits)d-%(M)dx%(N)dx%(K)d"
                                                      % c)
def test_mfma16_case(g, case):
    print("case:", case, flush=True)
    dtype, layout, M, N, K = case["dtype"], case["layout"], case["M"], case["N"], case["K"]
    a, b = inputs.make_operands(M, N, K, dtype, layout, DIST[dtype], seed=M * 5 + N * 11 + K)
    lda = K + case["pad"]
    ldb = (N if layout == "RR" else K) + case["pad"]
    ldc = (N + 3) // 4 * 4
    a_buf, a_ptr = place(a, lda, 0, dtype)
    b_buf, b_ptr = place(b, ldb, 0, dtype)
    info16, c16 = run(g, case, case["stages"], a_ptr, lda, b_ptr, ldb, ldc)
    info32, c32 = run(g, case, 1, a_ptr, lda, b_ptr, ldb, ldc)
    assert info16["mfma_block"] == 16 and info32["mfma_block"] == 32, (info16["mfma_block"], info32["mfma_block"])
    check_sentinel(c16, M, N, dtype)
    check_close(c16[:M, :N], oracle_full(a, b, dtype, layout), dtype, str(case))
    assert torch.equal(bits(c16[:M, :N]), bits(c32[:M, :N])), "16x16 and 32x32 blocks differ: %s" % case
    del a_buf, b_buf
