"""GPU parity of the stream-K entry point (gemm_run_streamk) against the oracle.

Small ragged shapes at every tile class, layout, dtype, stage count and
variant, with grids that cut tiles into pieces of every kind (a tile from
one workgroup, a tile summed from two or more, a workgroup's range ending
and starting inside one tile; workgroups numbered XCD by XCD when the grid
is a multiple of 8); for a fixed grid all (stages, variant) pairs
must agree bit for bit, since the pieces are whole units of the class's
largest K-tile and the partial tiles are added in K order.  Then shapes
whose tiles fill no whole number of rounds (the partial last wave stream-K
is for), against the oracle and against gemm_run (int8: the same bits),
data-parallel rounds followed by stream-K ones, and the workspace checks:
refusals leave C alone, and the arrival counters are zero after every call.
"""
import numpy as np
import pytest
import torch

import oracle
from software_pipelined_tiled_02_amd import binding, inputs
from tests.gpu_util import EPC, alloc_c, check_close, check_sentinel, oracle_full

pytestmark = pytest.mark.gpu

DTYPES = ("i8", "f16", "bf16", "f32")
LAYOUT_TILES = [("RC", "256x256"), ("RC", "256x256w8"), ("RC", "128x128"), ("RC", "32x64"),
                ("RR", "256x256"), ("RR", "256x256w8"), ("RR", "128x128"), ("RR", "32x64")]
DIST = {"i8": "int", "f16": "normal", "bf16": "uniform", "f32": "uniform"}


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gg = binding.Gemm(0)
    yield gg
    gg.close()


def run_sk(g, a, b, dtype, layout, stages, variant, M, N, K, grid, ldc=None):
    """gemm_run_streamk with the handle's workspace on device operands;
    returns (padded C on the CPU, the configuration used)."""
    ldb = N if layout == "RR" else K
    ldc = ldc or (N + 3) // 4 * 4
    c = alloc_c(M, N, ldc, dtype)
    _, info = binding.gemm_query_streamk(M, N, K, dtype, layout, stages, variant, grid=grid, tile=g.tile, ldc=ldc)
    g.run_streamk(M, N, K, dtype, layout, stages, variant, grid, a, K, b, ldb, c, ldc)
    torch.cuda.synchronize()
    return c.cpu(), info


def counters_zero(g):
    return int(g.workspace(65536)[:65536].count_nonzero()) == 0


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout,tile", LAYOUT_TILES)
def test_streamk_all_stages_variants(g, dtype, layout, tile):
    # 6 units of the 128x128 class's K-tile plus a ragged rest of three chunks;
    # N a multiple of 16 for layout RR, not of 4 for RC (masked column tail)
    M, N, K = 300, (144 if layout == "RR" else 138), 6 * 8 * EPC[dtype] + 3 * EPC[dtype]
    a, b = inputs.make_operands(M, N, K, dtype, layout, DIST[dtype], seed=31)
    ref = oracle_full(a, b, dtype, layout)
    ad, bd = a.cuda(), b.cuda()
    g.set_tile(tile)
    try:
        for grid in (2, 5, 16, 23):      # 16: workgroups numbered XCD by XCD
            first = None
            for stages in (1, 2, 3, 4):
                for variant in ("reg", "direct"):
                    what = "%s %s %s grid=%d S=%d %s" % (dtype, layout, tile, grid, stages, variant)
                    print("case:", what, flush=True)
                    c, info = run_sk(g, ad, bd, dtype, layout, stages, variant, M, N, K, grid)
                    assert info["sk_tiles"] > 0 and info["splits"] == 1, info
                    check_sentinel(c, M, N, dtype)
                    check_close(c[:M, :N], ref, dtype, what)
                    if first is None:
                        first = c
                    else:
                        assert torch.equal(c.view(torch.uint8), first.view(torch.uint8)), \
                            what + ": not bit-identical to S=1 reg"
            assert counters_zero(g), "arrival counters not back to zero"
    finally:
        g.set_tile("auto")


@pytest.mark.parametrize("dtype", ("i8", "bf16"))
def test_streamk_k_below_one_unit(g, dtype):
    """K shorter than one unit: every tile is one unit (its ragged head).
    15 tiles of 128x128 on a grid of 4: two rounds data-parallel, then 7
    tiles shared out over the 4 workgroups."""
    M, N, K = 520, 260, 3 * EPC[dtype]
    a, b = inputs.make_operands(M, N, K, dtype, "RC", DIST[dtype], seed=5)
    ref = oracle_full(a, b, dtype, "RC")
    g.set_tile("128x128")
    try:
        c, info = run_sk(g, a.cuda(), b.cuda(), dtype, "RC", 2, "reg", M, N, K, 4)
        assert info["grid"] == 4 and info["sk_tiles"] == 7, info
        check_sentinel(c, M, N, dtype)
        check_close(c[:M, :N], ref, dtype, "K below one unit")
    finally:
        g.set_tile("auto")


@pytest.mark.parametrize("dtype", ("i8", "f16"))
def test_streamk_after_data_parallel_rounds(g, dtype):
    """64 tiles of 128x128 on a grid of 14: three rounds data-parallel (every
    full round but the last), the remaining 22 tiles stream-K."""
    M, N, K = 1000, 1000, 1024 + 5 * EPC[dtype]
    a, b = inputs.make_operands(M, N, K, dtype, "RC", DIST[dtype], seed=9)
    ref = oracle_full(a, b, dtype, "RC")
    g.set_tile("128x128")
    try:
        first = None
        for stages, variant in ((2, "direct"), (3, "direct"), (1, "reg")):
            c, info = run_sk(g, a.cuda(), b.cuda(), dtype, "RC", stages, variant, M, N, K, 14)
            assert info["c_tiles"] == 64 and info["sk_tiles"] == 64 - 3 * 14 and info["grid"] == 14, info
            check_sentinel(c, M, N, dtype)
            check_close(c[:M, :N], ref, dtype, "DP + SK S=%d %s" % (stages, variant))
            if first is None:
                first = c
            else:
                assert torch.equal(c.view(torch.uint8), first.view(torch.uint8))
        assert counters_zero(g)
    finally:
        g.set_tile("auto")


@pytest.mark.parametrize("dtype", ("i8", "bf16"))
def test_streamk_unaligned_k(g, dtype):
    """The register-staged variant's ragged-K instances (K not whole 16-byte
    chunks) under stream-K."""
    M, N, K = 200, 96, 1501
    a, b = inputs.make_operands(M, N, K, dtype, "RC", DIST[dtype], seed=8)
    ref = oracle_full(a, b, dtype, "RC")
    ad, bd = a.cuda(), b.cuda()
    g.set_tile("128x128")
    try:
        first = None
        for stages in (1, 2, 3, 4):
            c, info = run_sk(g, ad, bd, dtype, "RC", stages, "reg", M, N, K, 3)
            assert info["sk_tiles"] > 0
            check_sentinel(c, M, N, dtype)
            check_close(c[:M, :N], ref, dtype, "%s K=%d S=%d stream-K" % (dtype, K, stages))
            if first is None:
                first = c
            else:
                assert torch.equal(c.view(torch.uint8), first.view(torch.uint8))
        assert counters_zero(g)
    finally:
        g.set_tile("auto")


@pytest.mark.parametrize("dtype", ("i8", "f32"))
def test_streamk_k_zero(g, dtype):
    """K = 0: every tile is one (empty) unit and C = 0."""
    M, N, K = 300, 200, 0
    a, b = inputs.make_operands(M, N, K, dtype, "RC", DIST[dtype], seed=1)
    c, info = run_sk(g, a.cuda(), b.cuda(), dtype, "RC", 2, "direct", M, N, K, 7)
    assert info["sk_tiles"] > 0 and info["grid"] <= 7, info
    check_sentinel(c, M, N, dtype)
    assert int(c[:M, :N].view(torch.uint8).count_nonzero()) == 0
    assert counters_zero(g)


# Partial last waves at full size, automatic tile and grid (one workgroup
# per CU): (M, N, K, dtype, dist, scale)
PARTIAL_WAVE = {
    "i8_4608x4608x4096": (4608, 4608, 4096, "i8", "int", 1.0),           # 324 tiles of 256x256
    "bf16_5120x5120x5128": (5120, 5120, 5128, "bf16", "uniform", 1.0),    # 400 tiles, ragged K
}


@pytest.mark.parametrize("name", list(PARTIAL_WAVE))
def test_streamk_partial_wave(g, name):
    M, N, K, dtype, dist, scale = PARTIAL_WAVE[name]
    print("workload:", name, flush=True)
    a, b = inputs.make_operands(M, N, K, dtype, "RC", dist, seed=12, scale=scale)
    ad, bd = a.cuda(), b.cuda()
    c_sk, info = run_sk(g, ad, bd, dtype, "RC", 3, "direct", M, N, K, 0, ldc=N)
    assert info["tile"] == binding.GEMM_TILE_256x256 and info["sk_tiles"] == info["c_tiles"], info
    assert info["grid"] == torch.cuda.get_device_properties(0).multi_processor_count or info["grid"] == 256
    check_sentinel(c_sk, M, N, dtype)
    c_dp = alloc_c(M, N, N, dtype)
    binding.gemm_run(g.h, M, N, K, dtype, "RC", 3, "direct", ad, K, bd, K, c_dp, N)
    torch.cuda.synchronize()
    c_dp = c_dp.cpu()
    if dtype == "i8":
        assert torch.equal(c_sk, c_dp), "stream-K int8 differs from gemm_run"
    # entries the oracle computes one by one: corners and two interior points of every tile, and edges
    rng = np.random.default_rng(3)
    rows, cols = [], []
    for m0 in range(0, M, 256):
        for n0 in range(0, N, 256):
            m1, n1 = min(M, m0 + 256) - 1, min(N, n0 + 256) - 1
            rows += [m0, m0, m1, m1] + list(rng.integers(m0, m1 + 1, 2))
            cols += [n0, n1, n0, n1] + list(rng.integers(n0, n1 + 1, 2))
    rows, cols = np.array(rows), np.array(cols)
    ref = oracle.gemm_entries(inputs.to_oracle(a, dtype), inputs.to_oracle(b, dtype), dtype, "RC", rows, cols)
    got = inputs.from_torch_out(c_sk[rows, cols], dtype)
    if dtype == "i8":
        assert np.array_equal(got, ref)
    else:
        rms = float(np.sqrt(np.mean(ref ** 2)))
        assert np.all(np.abs(got - ref) <= 1e-2 * np.abs(ref) + 1e-2 * rms), name
        # and against gemm_run's C everywhere: the same tolerance
        dp = inputs.from_torch_out(c_dp[:M, :N], dtype).astype(np.float64)
        sk = inputs.from_torch_out(c_sk[:M, :N], dtype).astype(np.float64)
        rms_dp = float(np.sqrt(np.mean(dp ** 2)))
        assert np.all(np.abs(sk - dp) <= 1e-2 * np.abs(dp) + 1e-2 * rms_dp), name
    assert counters_zero(g)


def test_streamk_workspace_errors(g):
    """A missing, short or misaligned workspace is refused and C is left alone."""
    M, N, K, dtype = 600, 600, 2048, "bf16"
    a, b = inputs.make_operands(M, N, K, dtype, "RC", DIST[dtype], seed=2)
    a, b = a.cuda(), b.cuda()
    c = alloc_c(M, N, N, dtype)
    _, info = binding.gemm_query_streamk(M, N, K, dtype, "RC", 2, "direct", grid=7, tile="auto")
    need = info["workspace_bytes"]
    assert info["sk_tiles"] > 0 and need > 0
    ws = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    run = lambda w, nbytes: binding.gemm_run_streamk(g.h, M, N, K, dtype, "RC", 2, "direct", 7, a, K, b, K,
                                                    c, N, w, nbytes, check=False)
    assert run(None, 0) == binding.GEMM_ERR_INVALID_ARG
    assert run(ws, need - 1) == binding.GEMM_ERR_INVALID_ARG
    assert run(ws.data_ptr() + 16, need) == binding.GEMM_ERR_ALIGNMENT
    torch.cuda.synchronize()
    check_sentinel(c.cpu(), 0, N, dtype)
    assert run(ws, need) == binding.GEMM_OK
    torch.cuda.synchronize()
    assert int(ws[:65536].count_nonzero()) == 0
