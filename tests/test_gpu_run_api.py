"""The binding's convenience call binding.run(A, B, ...) on torch tensors:
the same bits as gemm_run through the handle API (it is marshalling only),
with C allocated or given, on both layouts and every dtype, and against the
oracle."""
import pytest
import torch

from software_pipelined_tiled_02_amd import binding, inputs
from tests.gpu_util import check_close, oracle_full

pytestmark = pytest.mark.gpu

DIST = {"i8": "int", "f16": "normal", "bf16": "uniform", "f32": "uniform"}


@pytest.mark.parametrize("dtype", ("i8", "f16", "bf16", "f32"))
@pytest.mark.parametrize("layout", ("RC", "RR"))
def test_run_matches_gemm_run(dtype, layout):
    M, N, K = 300, 144, 528
    a, b = inputs.make_operands(M, N, K, dtype, layout, DIST[dtype], seed=17)
    ad, bd = a.cuda(), b.cuda()
    c1 = binding.run(ad, bd, layout=layout, stages=3, variant="direct")
    out = torch.full((M, N), 7, dtype=inputs.OUT_TORCH_DTYPES[dtype], device="cuda")
    c2 = binding.run(ad, bd, layout=layout, stages=2, variant="reg", out=out)
    assert c2 is out
    g = binding.Gemm(0)
    try:
        c3 = torch.empty((M, N), dtype=inputs.OUT_TORCH_DTYPES[dtype], device="cuda")
        g.run(ad, bd, c3, dtype, layout, 3, "direct")
    finally:
        g.close()
    torch.cuda.synchronize()
    assert c1.shape == (M, N) and c1.dtype == inputs.OUT_TORCH_DTYPES[dtype]
    assert torch.equal(c1.view(torch.uint8), c3.view(torch.uint8))
    assert torch.equal(c2.view(torch.uint8), c3.view(torch.uint8))      # every pair: the same bits
    check_close(c1.cpu(), oracle_full(a, b, dtype, layout), dtype, "binding.run %s %s" % (dtype, layout))


def test_run_on_a_side_stream():
    M, N, K = 256, 192, 384
    a, b = inputs.make_operands(M, N, K, "bf16", "RC", "uniform", seed=3)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = binding.run(a.cuda(), b.cuda())
    s.synchronize()
    check_close(c.cpu(), oracle_full(a, b, "bf16", "RC"), "bf16", "binding.run side stream")
