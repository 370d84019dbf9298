"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases span several tiles in M and N, a ragged edge in both, and a
ragged last K-tile, for every (dtype, layout, tile, stages, variant) the
library builds; the oracle computes them in full.  Closed-form cases
(identity, marker tiles) must be bit-exact at every dtype.  Full-size cases
(the benchmark workloads) compare sampled entries with the oracle.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from software_pipelined_tiled_02_amd import binding, inputs
from tests.gpu_util import EPC, check_close, check_sentinel, oracle_full, run_gpu

pytestmark = pytest.mark.gpu

DTYPES = ("i8", "f16", "bf16", "f32")
STAGES = (1, 2, 3, 4)
VARIANTS = ("reg", "direct")
# (layout, tile) pairs the library builds
LAYOUT_TILES = [("RC", "256x256"), ("RC", "256x256w8"), ("RC", "128x128"), ("RC", "32x64"),
                ("RR", "256x256"), ("RR", "256x256w8"), ("RR", "128x128"), ("RR", "32x64")]
DIST = {"i8": "int", "f16": "normal", "bf16": "uniform", "f32": "uniform"}
# K with a ragged last tile for every K-tile size of the dtype
SMALL_K = {"i8": 400, "f16": 200, "bf16": 200, "f32": 100}


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gg = binding.Gemm(0)
    yield gg
    gg.close()


def test_native_library_loaded():
    lib = binding.library()
    assert os.path.samefile(lib._name, binding.LIB_PATH)


_ref_cache = {}


def _small_case(dtype, layout, M=520, N=272, seed=3):
    K = SMALL_K[dtype]
    key = (dtype, layout, M, N, K, seed)
    if key not in _ref_cache:
        a, b = inputs.make_operands(M, N, K, dtype, layout, DIST[dtype], seed=seed)
        _ref_cache[key] = (a, b, oracle_full(a, b, dtype, layout))
    return (M, N, K) + _ref_cache[key]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout,tile", LAYOUT_TILES)
def test_small_all_stages_variants(g, dtype, layout, tile):
    """All 8 (stages, variant) pairs match the oracle and each other bit-for-bit."""
    M, N, K, a, b, ref = _small_case(dtype, layout)
    g.set_tile(tile)
    first = None
    for stages in STAGES:
        for variant in VARIANTS:
            what = "%s %s %s S=%d %s" % (dtype, layout, tile, stages, variant)
            print("case:", what, flush=True)
            c = run_gpu(g, a, b, dtype, layout, stages, variant, M, N, K)
            check_sentinel(c, M, N, dtype)
            check_close(c[:M, :N], ref, dtype, what)
            if first is None:
                first = c
            else:
                assert torch.equal(c.view(torch.uint8), first.view(torch.uint8)), \
                    what + ": not bit-identical to S=1 reg"
    g.set_tile("auto")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", ("RR", "RC"))
def test_padded_leading_dimensions(g, dtype, layout):
    M, N, K = 70, 48, 3 * EPC[dtype] * 4
    a, b = inputs.make_operands(M, N, K, dtype, layout, DIST[dtype], seed=11)
    ref = oracle_full(a, b, dtype, layout)
    e = EPC[dtype]
    for stages, variant in ((1, "direct"), (3, "reg"), (4, "direct")):
        c = run_gpu(g, a, b, dtype, layout, stages, variant, M, N, K,
                    lda=K + 2 * e, ldb=(N if layout == "RR" else K) + e, ldc=N + 4)
        check_sentinel(c, M, N, dtype)
        check_close(c[:M, :N], ref, dtype, "%s %s padded S=%d %s" % (dtype, layout, stages, variant))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", ("RR", "RC"))
@pytest.mark.parametrize("perm", (False, True))
def test_identity_is_exact(g, dtype, layout, perm):
    """A = I (or a permutation matrix) gives C = B (its rows permuted) exactly
    at every dtype: one nonzero term per sum."""
    K = 8 * EPC[dtype] * 4 + EPC[dtype]          # ragged last tile
    M, N = K, 96
    _, b = inputs.make_operands(1, N, K, dtype, layout, DIST[dtype], seed=5)
    a = torch.eye(M, K, dtype=torch.float32)
    if perm:
        a = a[torch.randperm(M, generator=torch.Generator().manual_seed(9))]
    a = a.to(inputs.TORCH_DTYPES[dtype]).contiguous()
    ref = oracle_full(a, b, dtype, layout)
    if perm:   # the oracle's C is B's rows permuted, with nothing added
        rows = torch.argmax(a.float(), dim=1).numpy()
        ref_b = oracle_full(torch.eye(K, K, dtype=torch.float32).to(inputs.TORCH_DTYPES[dtype]), b, dtype,
                            layout)
        assert np.array_equal(ref, ref_b[rows])
    for tile in ("auto", "128x128", "32x64"):
        g.set_tile(tile)
        for stages, variant in ((1, "reg"), (2, "direct"), (4, "direct"), (4, "reg")):
            c = run_gpu(g, a, b, dtype, layout, stages, variant, M, N, K)
            got = inputs.from_torch_out(c[:M, :N], dtype)
            assert np.array_equal(got, ref), (dtype, layout, tile, stages, variant)
    g.set_tile("auto")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout,tile", LAYOUT_TILES)
def test_marker_tiles(g, dtype, layout, tile):
    """A is zero except ones in K-tile t, B is all ones: C == (width of tile t)
    exactly, for every t including the ragged last one.  A stale or skipped
    ring slot shows up as 0 or twice the width."""
    _, info = binding.gemm_query(256, 128, 4096, dtype, layout, 4, "direct", tile=tile)
    for stages in STAGES:
        _, info = binding.gemm_query(64, 64, 64, dtype, layout, stages, "direct", tile=tile)
        bk = info["block_k"]
        K = (stages + 2) * bk + EPC[dtype]       # num_tiles = stages + 3, ragged tail
        nt = (K + bk - 1) // bk
        M, N = 64, 64
        tdt = inputs.TORCH_DTYPES[dtype]
        b = torch.ones((K, N) if layout == "RR" else (N, K), dtype=torch.float32).to(tdt)
        g.set_tile(tile)
        for t in range(nt):
            a = torch.zeros((M, K), dtype=torch.float32)
            a[:, t * bk: min(K, (t + 1) * bk)] = 1
            a = a.to(tdt)
            width = min(K, (t + 1) * bk) - t * bk
            for variant in VARIANTS:
                c = run_gpu(g, a, b, dtype, layout, stages, variant, M, N, K)
                got = inputs.from_torch_out(c[:M, :N], dtype)
                assert np.all(got == width), (dtype, layout, tile, stages, variant, t, np.unique(got))
    g.set_tile("auto")


@pytest.mark.parametrize("dtype", DTYPES)
def test_short_k_and_degenerate(g, dtype):
    """num_tiles in {1, 2, S-1, S, S+1}, K = 0, and tiny M, N."""
    for stages in STAGES:
        for variant in VARIANTS:
            _, info = binding.gemm_query(64, 64, 64, dtype, "RC", stages, variant, tile="128x128")
            bk = info["block_k"]
            for nt in sorted({1, 2, max(stages - 1, 1), stages, stages + 1}):
                K = nt * bk - (EPC[dtype] if nt > 1 else 0)
                M, N = 130, 36
                a, b = inputs.make_operands(M, N, K, dtype, "RC", DIST[dtype], seed=nt)
                ref = oracle_full(a, b, dtype, "RC")
                g.set_tile("128x128")
                c = run_gpu(g, a, b, dtype, "RC", stages, variant, M, N, K)
                check_sentinel(c, M, N, dtype)
                check_close(c[:M, :N], ref, dtype, "%s nt=%d S=%d %s" % (dtype, nt, stages, variant))
    g.set_tile("auto")
    # K = 0 writes zeros; M = 0 or N = 0 writes nothing
    for stages, variant in ((1, "reg"), (3, "direct")):
        a = torch.zeros((5, 0), dtype=inputs.TORCH_DTYPES[dtype]).cuda()
        b = torch.zeros((8, 0), dtype=inputs.TORCH_DTYPES[dtype]).cuda()
        from tests.gpu_util import alloc_c
        c = alloc_c(5, 8, 8, dtype)
        binding.gemm_run(g.h, 5, 8, 0, dtype, "RC", stages, variant, a, 16, b, 16, c, 8)
        torch.cuda.synchronize()
        assert bool((c[:5].float() == 0).all())
        check_sentinel(c.cpu(), 5, 8, dtype)
        c = alloc_c(0, 8, 8, dtype)
        binding.gemm_run(g.h, 0, 8, 16, dtype, "RC", stages, variant, None, 16, b, 16, c, 8)
        torch.cuda.synchronize()
        check_sentinel(c.cpu(), 0, 8, dtype)


def test_argument_errors_before_launch(g):
    a = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    bad = [
        dict(stages=0), dict(stages=5), dict(lda=32), dict(dtype=7), dict(layout=3), dict(variant=2),
    ]
    for kw in bad:
        args = dict(M=64, N=64, K=64, dtype="bf16", layout="RC", stages=2, variant="direct",
                    A=a, lda=64, B=a, ldb=64, C=c, ldc=64)
        args.update(kw)
        rc = binding.gemm_run(g.h, args["M"], args["N"], args["K"], args["dtype"], args["layout"],
                              args["stages"], args["variant"], args["A"], args["lda"], args["B"],
                              args["ldb"], args["C"], args["ldc"], check=False)
        assert rc == binding.GEMM_ERR_INVALID_ARG, kw
    rc = binding.gemm_run(g.h, 64, 64, 64, "bf16", "RC", 2, "direct", a.data_ptr() + 2, 64, a, 64,
                          c, 64, check=False)
    assert rc == binding.GEMM_ERR_ALIGNMENT
    rc = binding.gemm_run(g.h, 64, 64, 60, "bf16", "RC", 2, "direct", a, 64, a, 64, c, 64, check=False)
    assert rc == binding.GEMM_ERR_ALIGNMENT
