"""Helpers shared by the GPU tests: running the HIP path through the C ABI and
comparing it with the oracle at the tolerances the pages state.

Tolerances (the comparison is against the oracle's exact-input, double-
accumulated product):
  int8 -> int32 : bit-exact.
  fp16 / bf16   : |C - ref| <= 1e-2 * |ref| + 1e-2 * rms(ref) element-wise, and
                  ||C - ref||_F / ||ref||_F <= 1e-2.  This is the skill's fp16
                  tensor-core tolerance (abs 1e-2, rel 1e-2; "pipeline-gpu-kernel",
                  step 5) with the absolute term scaled by the result's rms so it
                  is independent of the input scale.
  fp32          : |C - ref| <= 1e-3 + 1e-3 * |ref| (the skill's FFMA tolerance).
"""
import numpy as np
import torch

import oracle
from software_pipelined_tiled_02_amd import binding, inputs

EPC = {"i8": 16, "f16": 8, "bf16": 8, "f32": 4}
SENTINEL = {"i8": 0x5A5A5A5A, "f16": 0x7E00, "bf16": 0x7FC0, "f32": 0x7FC00000}


def alloc_c(M, N, ldc, dtype):
    """C buffer of M + 2 rows of ldc, pre-filled with a sentinel bit pattern
    (the two extra rows catch stores past row M)."""
    out_dt = inputs.OUT_TORCH_DTYPES[dtype]
    itype = torch.int32 if out_dt in (torch.int32, torch.float32) else torch.int16
    c = torch.full((M + 2, max(ldc, 1)), 0, dtype=itype, device="cuda")
    pat = SENTINEL[dtype]
    if itype == torch.int16 and pat >= 0x8000:
        pat -= 0x10000
    if itype == torch.int32 and pat >= 0x80000000:
        pat -= 0x100000000
    c.fill_(pat)
    return c.view(out_dt)


def run_gpu(g, a_cpu, b_cpu, dtype, layout, stages, variant, M, N, K, lda=None, ldb=None, ldc=None):
    """Copy operands to the GPU (with optional padded leading dimensions), run
    the kernel, return the full padded C on the CPU."""
    lda = lda or K
    ldb = ldb or (N if layout == "RR" else K)
    ldc = ldc or N
    a = torch.zeros((max(M, 1), lda), dtype=a_cpu.dtype)
    a[:M, :K] = a_cpu
    b_rows = K if layout == "RR" else N
    b_cols = N if layout == "RR" else K
    b = torch.zeros((max(b_rows, 1), ldb), dtype=b_cpu.dtype)
    b[:b_rows, :b_cols] = b_cpu
    a, b = a.cuda(), b.cuda()
    c = alloc_c(M, N, ldc, dtype)
    binding.gemm_run(g.h, M, N, K, dtype, layout, stages, variant, a, lda, b, ldb, c, ldc)
    torch.cuda.synchronize()
    return c.cpu()


# Fill for the bytes around a placed operand: NaN for the float types, so a
# read of any byte past K or outside the rows shows up in C.
POISON = {"i8": 0x55, "f16": 0x7E00, "bf16": 0x7FC0, "f32": 0x7FC00000}


def place(t_cpu, ld, offset, dtype):
    """A CPU matrix (rows x cols, row-major) copied to the GPU with row
    stride `ld` elements, starting `offset` elements into a buffer that ends
    exactly at its last element; every other element holds POISON.
    Returns (buffer, device pointer of element (0, 0))."""
    rows, cols = t_cpu.shape
    n = offset + (rows - 1) * ld + cols if rows > 0 else offset
    itype = {1: torch.int8, 2: torch.int16, 4: torch.int32}[t_cpu.element_size()]
    pat = POISON[dtype]
    bits = 8 * t_cpu.element_size()
    if pat >= 1 << (bits - 1):
        pat -= 1 << bits
    flat = torch.full((max(n, 1),), pat, dtype=itype)
    raw = t_cpu.contiguous().view(itype)
    for r in range(rows):
        flat[offset + r * ld: offset + r * ld + cols] = raw[r]
    buf = flat.cuda()
    return buf, buf.data_ptr() + offset * t_cpu.element_size()


def run_gpu_placed(g, a_cpu, b_cpu, dtype, layout, stages, variant, M, N, K, lda, ldb, offset,
                   check=True):
    """run_gpu with A and B placed by `place` (row strides lda / ldb, both
    `offset` elements into their buffers).  Returns (status, padded C)."""
    a_buf, a_ptr = place(a_cpu, lda, offset, dtype)
    b_buf, b_ptr = place(b_cpu, ldb, offset, dtype)
    c = alloc_c(M, N, N, dtype)
    rc = binding.gemm_run(g.h, M, N, K, dtype, layout, stages, variant, a_ptr, lda, b_ptr, ldb, c, N,
                          check=check)
    torch.cuda.synchronize()
    del a_buf, b_buf
    return rc, c.cpu()


def run_gpu_splitk(g, a_cpu, b_cpu, dtype, layout, stages, variant, M, N, K, splits):
    """run_gpu through gemm_run_splitk with the handle's workspace; returns
    (padded C on the CPU, the configuration used)."""
    ldb = N if layout == "RR" else K
    ldc = (N + 3) // 4 * 4                    # C rows: whole 16-byte groups of 4-byte words
    a, b = a_cpu.cuda(), b_cpu.cuda()
    c = alloc_c(M, N, ldc, dtype)
    _, info = binding.gemm_query(M, N, K, dtype, layout, stages, variant, tile=g.tile, ldc=ldc, splits=splits)
    g.run_splitk(M, N, K, dtype, layout, stages, variant, splits, a, K, b, ldb, c, ldc)
    torch.cuda.synchronize()
    return c.cpu(), info


def oracle_full(a_cpu, b_cpu, dtype, layout):
    return oracle.gemm(inputs.to_oracle(a_cpu, dtype), inputs.to_oracle(b_cpu, dtype), dtype, layout)


def oracle_full_widened(a_cpu, b_cpu, dtype, layout):
    """oracle_full for large fp16/bf16 shapes through the oracle's fp32
    entry: every fp16 and bf16 value is exactly an fp32 value (torch's
    widening is exact), and the oracle decodes both encodings exactly to
    double and then does the same double arithmetic in the same k order, so
    the result is the same doubles, bit for bit (pinned on the CPU by
    tests/test_oracle.py) -- only the per-element decoding, which dominates
    the oracle's time for fp16, is skipped.  Other dtypes: oracle_full."""
    if dtype not in ("f16", "bf16"):
        return oracle_full(a_cpu, b_cpu, dtype, layout)
    return oracle.gemm(a_cpu.float().contiguous().numpy(), b_cpu.float().contiguous().numpy(), "f32", layout)


def check_close(c_gpu, ref, dtype, what=""):
    """Assert the pages' tolerance for dtype; returns (max_abs_err, frob_rel)."""
    got = inputs.from_torch_out(c_gpu, dtype)
    if dtype == "i8":
        bad = np.argwhere(got != ref)
        assert bad.size == 0, "%s: %d int mismatches, first at %s (%d vs %d)" % (
            what, len(bad), bad[0], got[tuple(bad[0])], ref[tuple(bad[0])])
        return 0.0, 0.0
    d = np.abs(got - ref)
    if dtype == "f32":
        tol = 1e-3 + 1e-3 * np.abs(ref)
    else:
        rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
        tol = 1e-2 * np.abs(ref) + 1e-2 * rms
    bad = np.argwhere(~(d <= tol))
    assert bad.size == 0, "%s: %d elements out of tolerance, first at %s (%r vs %r)" % (
        what, len(bad), bad[0], got[tuple(bad[0])], ref[tuple(bad[0])])
    nref = float(np.linalg.norm(ref))
    frob = float(np.linalg.norm(got - ref)) / nref if nref > 0 else float(np.linalg.norm(got))
    if dtype != "f32":
        assert frob <= 1e-2, "%s: Frobenius relative error %g" % (what, frob)
    return float(d.max()) if d.size else 0.0, frob


def check_sentinel(c_pad, M, N, dtype):
    """Everything of the padded C outside rows < M, columns < N must still
    hold the sentinel."""
    out_dt = c_pad.dtype
    itype = torch.int32 if out_dt in (torch.int32, torch.float32) else torch.int16
    pat = SENTINEL[dtype]
    if itype == torch.int16 and pat >= 0x8000:
        pat -= 0x10000
    if itype == torch.int32 and pat >= 0x80000000:
        pat -= 0x100000000
    raw = c_pad.contiguous().view(itype)
    assert bool((raw[M:] == pat).all()), "kernel wrote past row M"
    if raw.shape[1] > N and M > 0:
        assert bool((raw[:M, N:] == pat).all()), "kernel wrote past column N"
