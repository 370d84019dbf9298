"""GPU check of gemm_run_splitk_noalloc, the entry point that allocates
nothing: its split-K workspace is the library's static scratch array.

Through the C ABI it must give C bit for bit equal to gemm_run_splitk with a
caller workspace (same kernels, same split count), and both must meet the
oracle's tolerance, on two calls in a row, the second with a smaller input
(the scratch keeps the last call's contents; its counters must be zero
again after every call).  A call needing more than the scratch size is
refused before any HIP call.
"""
import pytest
import torch

from software_pipelined_tiled_02_amd import binding, inputs
from tests.gpu_util import EPC, alloc_c, check_close, check_sentinel, oracle_full

pytestmark = pytest.mark.gpu

DIST = {"i8": "int", "f16": "normal", "bf16": "uniform", "f32": "uniform"}


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gg = binding.Gemm(0)
    yield gg
    gg.close()


def _run_both(g, dtype, layout, tile, stages, variant, splits, M, N, K, seed):
    a, b = inputs.make_operands(M, N, K, dtype, layout, DIST[dtype], seed=seed)
    ldb = N if layout == "RR" else K
    ldc = -(-N // 4) * 4
    _, info = binding.gemm_query(M, N, K, dtype, layout, stages, variant, tile=tile, ldc=ldc, splits=splits)
    assert 0 < info["workspace_bytes"] <= binding.GEMM_NOALLOC_SCRATCH_BYTES, info
    ad, bd = a.cuda(), b.cuda()
    c_ws = alloc_c(M, N, ldc, dtype)
    c_na = alloc_c(M, N, ldc, dtype)
    ws = g.workspace(info["workspace_bytes"])
    binding.gemm_run_splitk(g.h, M, N, K, dtype, layout, stages, variant, splits, ad, K, bd, ldb, c_ws, ldc,
                            ws, ws.numel())
    binding.gemm_run_splitk_noalloc(g.h, M, N, K, dtype, layout, stages, variant, splits, ad, K, bd, ldb,
                                    c_na, ldc)
    torch.cuda.synchronize()
    return a, b, c_ws.cpu(), c_na.cpu(), info


# (dtype, layout, tile, stages, variant, splits, (M, N, K) of the first call, of the second)
CASES = [
    ("bf16", "RC", "128x128", 2, "direct", 0, (1024, 512, 4096 + 16), (300, 138, 6 * 64 + 24)),
    ("i8", "RC", "256x256", 3, "direct", 4, (512, 768, 8 * 128 + 48), (260, 200, 4 * 128 + 16)),
    ("f16", "RR", "32x64", 4, "reg", 5, (600, 256, 2048 + 8), (100, 64, 6 * 128 + 8)),
    ("f32", "RC", "128x128", 1, "reg", 3, (700, 300, 1024 + 4), (129, 130, 3 * 32 + 4)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_%s_%s_S%d_%s" % c[:5])
def test_noalloc_matches_workspace_entry(g, case):
    dtype, layout, tile, stages, variant, splits, big, small = case
    g.set_tile(tile)
    try:
        for call, (M, N, K) in enumerate((big, small)):
            if layout == "RR":
                N = -(-N // EPC[dtype]) * EPC[dtype]
            what = "%s %s %s S=%d %s splits=%d %dx%dx%d (call %d)" % (
                dtype, layout, tile, stages, variant, splits, M, N, K, call)
            print("case:", what, flush=True)
            a, b, c_ws, c_na, info = _run_both(g, dtype, layout, tile, stages, variant, splits, M, N, K,
                                               seed=31 + call)
            assert info["splits"] > 1, info
            assert torch.equal(c_na.view(torch.uint8), c_ws.view(torch.uint8)), what + ": differs from gemm_run_splitk"
            check_sentinel(c_na, M, N, dtype)
            check_close(c_na[:M, :N], oracle_full(a, b, dtype, layout), dtype, what)
    finally:
        g.set_tile("auto")


def test_noalloc_refuses_over_the_scratch_size(g):
    # 8192 x 8192 with two K splits of 256x256 tiles needs 512 MiB of partials
    M = N = 8192
    K = 1024
    _, info = binding.gemm_query(M, N, K, "bf16", "RC", 2, "direct", splits=2)
    assert info["workspace_bytes"] > binding.GEMM_NOALLOC_SCRATCH_BYTES
    c = torch.empty(16, dtype=torch.bfloat16, device="cuda")   # never written: the call is refused first
    rc = binding.gemm_run_splitk_noalloc(g.h, M, N, K, "bf16", "RC", 2, "direct", 2, c, K, c, K, c, N,
                                         check=False)
    assert rc == binding.GEMM_ERR_SCRATCH
    assert "GEMM_NOALLOC_SCRATCH_BYTES" in binding.gemm_status_string(rc)


def test_noalloc_single_split_uses_no_scratch(g):
    """With one split the call is plain gemm_run: same bits."""
    M, N, K = 300, 144, 6 * 64 + 8
    a, b = inputs.make_operands(M, N, K, "bf16", "RC", "uniform", seed=5)
    ad, bd = a.cuda(), b.cuda()
    c1 = alloc_c(M, N, N, "bf16")
    c2 = alloc_c(M, N, N, "bf16")
    binding.gemm_run(g.h, M, N, K, "bf16", "RC", 2, "direct", ad, K, bd, K, c1, N)
    binding.gemm_run_splitk_noalloc(g.h, M, N, K, "bf16", "RC", 2, "direct", 1, ad, K, bd, K, c2, N)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.uint8), c2.view(torch.uint8))
