"""GPU parity at the benchmark workloads' full sizes, in the launch
configuration the benchmark times (automatic tile choice, every stage count
and load variant).

The two 4096^3 workloads of the benchmark's headline sweep (int8 and fp16,
layout RC) and both tile-loop shapes are compared in full, element by
element, with the whole oracle product.  The others are compared on sampled
entries the oracle computes one by one: every C tile of the launched tile
size contributes its four corners and two interior points, and every edge
row and column is sampled.  Within a workload every (stages, variant) pair
must agree with the first bit for bit, since pipelining only reorders loads
("pipeline-gpu-kernel", step 5).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from software_pipelined_tiled_02_amd import binding, inputs
from tests.gpu_util import alloc_c, check_close, check_sentinel, oracle_full_widened

pytestmark = pytest.mark.gpu

ALL_PAIRS = [(s, v) for s in (1, 2, 3, 4) for v in ("reg", "direct")]
# The best pair first: it is the one compared with the oracle in full.
BEST_FIRST = [(3, "direct")] + [p for p in ALL_PAIRS if p != (3, "direct")]
# name: (M, N, K, dtype, layout, dist, scale, compare the whole C)
WORKLOADS = {
    "fp32_256_rr": (256, 256, 256, "f32", "RR", "uniform", 1.0, True),
    "int8_4096_rc": (4096, 4096, 4096, "i8", "RC", "int", 1.0, True),
    "fp16_4096_rc": (4096, 4096, 4096, "f16", "RC", "normal", 1.0 / 64.0, True),
    "bf16_skinny_8192x64x8192": (8192, 64, 8192, "bf16", "RC", "normal", 1.0, False),
    "bf16_8192x8192x8200": (8192, 8192, 8200, "bf16", "RC", "uniform", 1.0, False),
    # layout RR at the 256x256 tile (B fragments by transposing LDS reads)
    "fp16_4096_rr": (4096, 4096, 4096, "f16", "RR", "normal", 1.0 / 64.0, False),
    "int8_4096_rr": (4096, 4096, 4096, "i8", "RR", "int", 1.0, False),
    # the fp32 comparison at a compute-bound size (B element reads)
    "fp32_4096_rr": (4096, 4096, 4096, "f32", "RR", "uniform", 1.0, False),
}


@pytest.fixture(scope="module")
def g():
    gg = binding.Gemm(0)
    yield gg
    gg.close()


def sample_points(M, N, bm, bn, n, seed):
    """Entries to check: the four corners and two random interior points of
    every bm x bn tile of C, the four corners of C, 8 points on each edge
    row and column, and n random points."""
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    for m0 in range(0, M, bm):
        m1 = min(M, m0 + bm) - 1
        for n0 in range(0, N, bn):
            n1 = min(N, n0 + bn) - 1
            rows += [m0, m0, m1, m1] + list(rng.integers(m0, m1 + 1, 2))
            cols += [n0, n1, n0, n1] + list(rng.integers(n0, n1 + 1, 2))
    rows += list(rng.integers(0, M, n)) + [0, 0, M - 1, M - 1] + [M - 1] * 8 + list(rng.integers(0, M, 8))
    cols += list(rng.integers(0, N, n)) + [0, N - 1, 0, N - 1] + list(rng.integers(0, N, 8)) + [N - 1] * 8
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def check_samples(got, ref, dtype, rms, what):
    if dtype == "i8":
        assert np.array_equal(got, ref), what
        return
    d = np.abs(got - ref)
    if dtype == "f32":
        tol = 1e-3 + 1e-3 * np.abs(ref)
    else:
        tol = 1e-2 * np.abs(ref) + 1e-2 * rms
    assert np.all(d <= tol), (what, float(d.max()))
    assert np.linalg.norm(got - ref) <= 1e-2 * np.linalg.norm(ref), what


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload(g, name):
    M, N, K, dtype, layout, dist, scale, full = WORKLOADS[name]
    print("workload:", name, "full" if full else "sampled", flush=True)
    a, b = inputs.make_operands(M, N, K, dtype, layout, dist, seed=0, scale=scale)
    ad, bd = a.cuda(), b.cuda()
    ldb = N if layout == "RR" else K
    if full:
        ref = oracle_full_widened(a, b, dtype, layout)
    else:
        _, info = binding.gemm_query(M, N, K, dtype, layout, 2, "direct")
        rows, cols = sample_points(M, N, info["block_m"], info["block_n"], 3000, seed=1)
        ref = oracle.gemm_entries(inputs.to_oracle(a, dtype), inputs.to_oracle(b, dtype), dtype, layout,
                                  rows, cols)
        rms = float(np.sqrt(np.mean(ref ** 2)))
    first = None
    for stages, variant in BEST_FIRST:
        what = "%s S=%d %s" % (name, stages, variant)
        print("  stages=%d variant=%s" % (stages, variant), flush=True)
        c = alloc_c(M, N, N, dtype)
        binding.gemm_run(g.h, M, N, K, dtype, layout, stages, variant, ad, K, bd, ldb, c, N)
        torch.cuda.synchronize()
        if first is None:
            # the first pair against the oracle: every element, or the samples
            if full:
                check_close(c[:M].cpu(), ref, dtype, what)
            else:
                check_samples(inputs.from_torch_out(c[rows, cols], dtype), ref, dtype, rms, what)
            check_sentinel(c[M:], 0, N, dtype)
            first = c
        else:
            # every other pair: the same bits as the first (and so the same
            # comparison with the oracle)
            assert torch.equal(c.view(torch.uint8), first.view(torch.uint8)), \
                "%s differs bitwise from S=3 direct" % what
        del c
    del first
    torch.cuda.empty_cache()


# More 256x256 tiles than CUs, so each workgroup loops over several tiles,
# with ragged M, N and K edges: (M, N, K, dtype, dist, scale); compared in
# full with the oracle.
PERSISTENT = {
    "bf16_4100x4200x1000": (4100, 4200, 1000, "bf16", "uniform", 1.0),
    "i8_4300x4120x1008": (4300, 4120, 1008, "i8", "int", 1.0),
}


@functools.lru_cache(maxsize=None)
def _persistent_case(name):
    M, N, K, dtype, dist, scale = PERSISTENT[name]
    a, b = inputs.make_operands(M, N, K, dtype, "RC", dist, seed=3, scale=scale)
    return a, b, oracle_full_widened(a, b, dtype, "RC")


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
        a, b, ref = _persistent_case(name)
        ad, bd = a.cuda(), b.cuda()
        first = None
        for stages, variant in [(2, "direct"), (3, "direct"), (1, "direct"), (3, "reg"), (4, "direct"),
                                (1, "reg"), (2, "reg"), (4, "reg")]:
            what = "%s %s S=%d %s" % (name, tile, stages, variant)
            print("  stages=%d variant=%s" % (stages, variant), flush=True)
            c = alloc_c(M, N, N, dtype)
            binding.gemm_run(gg.h, M, N, K, dtype, "RC", stages, variant, ad, K, bd, K, c, N)
            torch.cuda.synchronize()
            if first is None:
                check_close(c[:M].cpu(), ref, dtype, what)
                check_sentinel(c[M:], 0, N, dtype)
                first = c
            else:
                assert torch.equal(c.view(torch.uint8), first.view(torch.uint8)), what
    finally:
        gg.close()
    torch.cuda.empty_cache()
