"""GPU parity at the benchmark workloads' full sizes, in the launch
configuration the benchmark times (automatic tile choice, each stage count
and load variant).  The oracle computes sampled entries one by one (every
corner and edge row/column included); all (stages, variant) pairs must also
agree bit-for-bit, since pipelining only reorders loads.
"""
import numpy as np
import pytest
import torch

import oracle
from software_pipelined_tiled_02_amd import binding, inputs
from tests.gpu_util import alloc_c, check_sentinel

pytestmark = pytest.mark.gpu

# name: (M, N, K, dtype, layout, dist, scale, pairs)
ALL_PAIRS = [(s, v) for s in (1, 2, 3, 4) for v in ("reg", "direct")]
WORKLOADS = {
    "fp32_256_rr": (256, 256, 256, "f32", "RR", "uniform", 1.0, ALL_PAIRS),
    "int8_4096_rc": (4096, 4096, 4096, "i8", "RC", "int", 1.0, ALL_PAIRS),
    "fp16_4096_rc": (4096, 4096, 4096, "f16", "RC", "normal", 1.0 / 64.0, ALL_PAIRS),
    "bf16_skinny_8192x64x8192": (8192, 64, 8192, "bf16", "RC", "normal", 1.0, ALL_PAIRS),
    "bf16_8192x8192x8200": (8192, 8192, 8200, "bf16", "RC", "uniform", 1.0,
                            [(3, "direct"), (4, "direct"), (4, "reg"), (2, "direct"), (1, "direct")]),
    # layout RR at the 256x256 tile (B fragments by transposing LDS reads)
    "fp16_4096_rr": (4096, 4096, 4096, "f16", "RR", "normal", 1.0 / 64.0,
                     [(3, "direct"), (2, "direct"), (2, "reg"), (4, "direct"), (1, "direct"), (3, "reg")]),
    "int8_4096_rr": (4096, 4096, 4096, "i8", "RR", "int", 1.0,
                     [(3, "direct"), (2, "direct"), (2, "reg"), (4, "direct"), (1, "reg")]),
}


@pytest.fixture(scope="module")
def g():
    gg = binding.Gemm(0)
    yield gg
    gg.close()


def sample_points(M, N, n, seed):
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, n)) + [0, 0, M - 1, M - 1] + [M - 1] * 8 + list(rng.integers(0, M, 8))
    cols = list(rng.integers(0, N, n)) + [0, N - 1, 0, N - 1] + list(rng.integers(0, N, 8)) + [N - 1] * 8
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload(g, name):
    M, N, K, dtype, layout, dist, scale, pairs = WORKLOADS[name]
    print("workload:", name, flush=True)
    a, b = inputs.make_operands(M, N, K, dtype, layout, dist, seed=0, scale=scale)
    rows, cols = sample_points(M, N, 3000, seed=1)
    ref = oracle.gemm_entries(inputs.to_oracle(a, dtype), inputs.to_oracle(b, dtype), dtype, layout,
                              rows, cols)
    ad, bd = a.cuda(), b.cuda()
    ldb = N if layout == "RR" else K
    first = None
    rms = None
    for stages, variant in pairs:
        print("  stages=%d variant=%s" % (stages, variant), flush=True)
        c = alloc_c(M, N, N, dtype)
        binding.gemm_run(g.h, M, N, K, dtype, layout, stages, variant, ad, K, bd, ldb, c, N)
        torch.cuda.synchronize()
        got = inputs.from_torch_out(c[rows, cols], dtype)
        if dtype == "i8":
            assert np.array_equal(got, ref), (name, stages, variant)
        else:
            if rms is None:
                rms = float(np.sqrt(np.mean(ref ** 2)))
            d = np.abs(got - ref)
            if dtype == "f32":
                tol = 1e-3 + 1e-3 * np.abs(ref)
            else:
                tol = 1e-2 * np.abs(ref) + 1e-2 * rms
            assert np.all(d <= tol), (name, stages, variant, float(d.max()))
            assert np.linalg.norm(got - ref) <= 1e-2 * np.linalg.norm(ref), (name, stages, variant)
        check_sentinel(c[M:], 0, N, dtype)
        if first is None:
            first = c
        else:
            assert torch.equal(c.view(torch.uint8), first.view(torch.uint8)), \
                "%s S=%d %s differs bitwise from the first pair" % (name, stages, variant)
        del c
    torch.cuda.empty_cache()


# More 256x256 tiles than CUs, so each workgroup loops over several tiles,
# with ragged M, N and K edges: (M, N, K, dtype, dist, scale)
PERSISTENT = {
    "bf16_4100x4200x1000": (4100, 4200, 1000, "bf16", "uniform", 1.0),
    "i8_4300x4120x1008": (4300, 4120, 1008, "i8", "int", 1.0),
}


@pytest.mark.parametrize("tile", ["256x256", "256x256w8"])
@pytest.mark.parametrize("name", list(PERSISTENT))
def test_tile_loop_with_edges(name, tile):
    M, N, K, dtype, dist, scale = PERSISTENT[name]
    print("workload:", name, tile, flush=True)
    gg = binding.Gemm(0)
    try:
        gg.set_tile(tile)
        _, info = binding.gemm_query(M, N, K, dtype, "RC", 2, "direct", tile=tile)
        assert info["c_tiles"] > info["grid"] == 256, info
        a, b = inputs.make_operands(M, N, K, dtype, "RC", dist, seed=3, scale=scale)
        rows, cols = sample_points(M, N, 3000, seed=4)
        ref = oracle.gemm_entries(inputs.to_oracle(a, dtype), inputs.to_oracle(b, dtype), dtype, "RC",
                                  rows, cols)
        ad, bd = a.cuda(), b.cuda()
        first = None
        for stages, variant in [(2, "direct"), (3, "direct"), (1, "direct"), (3, "reg"), (4, "direct")]:
            print("  stages=%d variant=%s" % (stages, variant), flush=True)
            c = alloc_c(M, N, N, dtype)
            binding.gemm_run(gg.h, M, N, K, dtype, "RC", stages, variant, ad, K, bd, K, c, N)
            torch.cuda.synchronize()
            got = inputs.from_torch_out(c[rows, cols], dtype)
            if dtype == "i8":
                assert np.array_equal(got, ref), (name, stages, variant)
            else:
                rms = float(np.sqrt(np.mean(ref ** 2)))
                assert np.all(np.abs(got - ref) <= 1e-2 * np.abs(ref) + 1e-2 * rms), (name, stages, variant)
            check_sentinel(c[M:], 0, N, dtype)
            if first is None:
                first = c
            else:
                assert torch.equal(c.view(torch.uint8), first.view(torch.uint8)), (name, stages, variant)
    finally:
        gg.close()
    torch.cuda.empty_cache()
