"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and its argument checks and configuration choice behave as the
header says -- all through gemm_query, which makes no HIP call.
"""
import re

import pytest

from software_pipelined_tiled_02_amd import binding
from tests.conftest import ROOT

HEADER = ROOT + "/include/pipegemm.h"


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gemm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_function():
    lib = binding.library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def q(M=4096, N=4096, K=4096, dtype="bf16", layout="RC", stages=2, variant="direct", tile="auto", **kw):
    return binding.gemm_query(M, N, K, dtype, layout, stages, variant, tile=tile, check=False, **kw)


def test_invalid_arguments():
    E = binding.GEMM_ERR_INVALID_ARG
    assert q(stages=0)[0] == E
    assert q(stages=5)[0] == E
    assert q(dtype=9)[0] == E
    assert q(layout=2)[0] == E
    assert q(variant=3)[0] == E
    assert q(M=-1)[0] == E
    assert q(K=-16)[0] == E
    assert q(lda=4000)[0] == E          # lda < K
    assert q(ldb=100)[0] == E           # RC: ldb < K
    assert q(layout="RR", ldb=100)[0] == E  # RR: ldb < N
    assert q(ldc=10)[0] == E
    assert q(tile=7)[0] == E


def test_alignment():
    A = binding.GEMM_ERR_ALIGNMENT
    assert q(K=4100)[0] == A                      # K*2 B not a multiple of 16
    assert q(dtype="i8", K=4104)[0] == A          # i8: K % 16
    assert q(dtype="f32", K=4098)[0] == A
    assert q(lda=4100)[0] == A                    # lda*2 B
    assert q(ldb=4100)[0] == A                    # RC: ldb*2 B
    assert q(ldc=4098)[0] == A                    # ldc % 4
    assert q(A=8)[0] == A                         # pointer not 16-byte aligned
    assert q(layout="RR", N=4100)[0] == A         # RR: N % 8
    assert q(K=8200)[0] == binding.GEMM_OK        # 8200 * 2 B = 1025 * 16 B


def test_register_staged_takes_unaligned_rows():
    """The register-staged variant takes any K and leading dimension and
    16-byte-unaligned operand pointers; C's rules and RR's N rule stay."""
    A, OK = binding.GEMM_ERR_ALIGNMENT, binding.GEMM_OK
    for stages in (1, 2, 3, 4):
        assert q(K=4100, variant="reg", stages=stages)[0] == OK
        assert q(dtype="i8", K=4097, lda=4099, variant="reg", stages=stages)[0] == OK
        assert q(dtype="f32", K=4098, variant="reg", stages=stages)[0] == OK
        assert q(layout="RR", K=1001, ldb=4104, variant="reg", stages=stages)[0] == OK
    assert q(lda=4100, ldb=4098, variant="reg")[0] == OK
    assert q(A=8, B=24, variant="reg")[0] == OK
    assert q(dtype="i8", A=9, B=3, variant="reg")[0] == OK
    assert q(A=9, variant="reg")[0] == A          # bf16: pointer not element-aligned
    assert q(dtype="f32", B=6, variant="reg")[0] == A
    assert q(ldc=4098, variant="reg")[0] == A     # C keeps its 16-byte rows
    assert q(layout="RR", N=4100, variant="reg")[0] == A
    rc, info = q(K=1001, variant="reg")
    assert rc == OK and info["k_tiles"] == -(-1001 // info["block_k"]) and info["k_tail"] == 1001 % info["block_k"]


def test_unsupported():
    U = binding.GEMM_ERR_UNSUPPORTED
    assert q(layout="RR", tile="256x256")[0] == binding.GEMM_OK   # every tile class has both layouts
    assert q(M=2 ** 31)[0] == U
    assert q(lda=2 ** 23, K=64)[0] == U           # 256 rows * 16 MiB > 2^31 B


def test_empty_sizes_are_valid():
    rc, info = q(M=0)
    assert rc == binding.GEMM_OK and info["grid"] == 0
    rc, info = q(K=0)
    assert rc == binding.GEMM_OK and info["k_tiles"] == 0


@pytest.mark.parametrize("dtype,bk2,bk4", [("bf16", 64, 32), ("f16", 64, 32), ("i8", 128, 64), ("f32", 32, 16)])
def test_large_tile_budget(dtype, bk2, bk4):
    """256x256 tiles: the K-tile halves where the ring would not fit 160 KiB
    (4 stages, and 3 register-staged stages); the 3-stage direct ring keeps
    it and splits by operand: three A slots and two B slots, 160 KiB."""
    sz = {"bf16": 2, "f16": 2, "i8": 1, "f32": 4}[dtype]
    for stages in (1, 2, 3, 4):
        for variant in ("reg", "direct"):
            rc, info = q(dtype=dtype, stages=stages, variant=variant, tile="256x256")
            assert rc == binding.GEMM_OK
            split = stages == 3 and variant == "direct"
            bk = bk2 if stages <= 2 or split else bk4
            assert info["block_k"] == bk
            slots = stages if variant == "direct" else min(stages, 2)
            assert info["lds_slots"] == slots
            ring = (3 * 256 + 2 * 256) * bk * sz if split else slots * (256 + 256) * bk * sz
            assert not split or ring == 160 * 1024
            # the epilogue stages 32 rows of each wave's 128-column block of C
            # (4-byte outputs for int8/fp32, rows padded by 16 B; 2-byte for
            # fp16/bf16, rows padded by 32 B)
            strips = 4 * 32 * (128 * 4 + 16 if dtype in ("i8", "f32") else 128 * 2 + 32)
            assert info["lds_bytes"] == max(ring, strips) <= 160 * 1024
            # the 8-wave 256x256 tile: the same ring, 8 strips of 64-column blocks
            rc, w8 = q(dtype=dtype, stages=stages, variant=variant, tile="256x256w8")
            assert rc == binding.GEMM_OK and w8["threads"] == 512 and w8["block_k"] == bk
            strips8 = 8 * 32 * (64 * 4 + 16 if dtype in ("i8", "f32") else 64 * 2 + 32)
            assert w8["lds_bytes"] == max(ring, strips8) <= 160 * 1024
            assert info["reg_sets"] == (0 if variant == "direct" else max(1, stages - 1))
            assert info["tiles_in_flight"] == (stages - 1 if variant == "direct" else max(1, stages - 1))


def test_mfma_block_shape():
    """16x16 MFMA blocks exactly for the 4-wave 256x256 tile's 2-3 stage
    direct rings with int8/fp16/bf16 (both layouts); 32x32 everywhere else."""
    for dtype in ("i8", "f16", "bf16", "f32"):
        for layout in ("RC", "RR"):
            for tile in ("256x256", "256x256w8", "128x128", "32x64"):
                for stages in (1, 2, 3, 4):
                    for variant in ("reg", "direct"):
                        rc, info = q(dtype=dtype, layout=layout, stages=stages, variant=variant, tile=tile)
                        if rc != binding.GEMM_OK:
                            continue
                        want16 = (tile == "256x256" and variant == "direct" and stages in (2, 3) and
                                  dtype != "f32")
                        assert info["mfma_block"] == (16 if want16 else 32), (dtype, layout, tile, stages, variant)


def test_auto_tile_choice():
    assert q()[1]["tile"] == binding.GEMM_TILE_256x256                # 256 tiles of 256x256
    assert q(M=8192, N=64, K=8192)[1]["tile"] == binding.GEMM_TILE_32x64
    assert q(M=2048, N=2048)[1]["tile"] == binding.GEMM_TILE_128x128  # 64 big tiles < 256 CUs
    assert q(dtype="f32", layout="RR", M=256, N=256, K=256)[1]["tile"] == binding.GEMM_TILE_32x64
    assert q(layout="RR")[1]["tile"] == binding.GEMM_TILE_256x256
    info = q(M=8192, N=8192, K=8200, stages=4)[1]
    assert info["tile"] == binding.GEMM_TILE_256x256 and info["threads"] == 256
    w8 = q(M=8192, N=8192, K=8200, stages=4, tile="256x256w8")[1]
    assert (w8["tile"], w8["threads"], w8["grid"]) == (binding.GEMM_TILE_256x256_W8, 512, 256)
    assert (info["c_tiles"], info["k_tiles"], info["k_tail"], info["block_k"]) == (1024, 257, 8, 32)
    assert info["grid"] == 256          # one workgroup per CU, four tiles each
    assert q()[1]["grid"] == q()[1]["c_tiles"] == 256


def test_status_strings():
    for s in range(6):
        assert binding.gemm_status_string(s).startswith("GEMM_")
    assert binding.gemm_status_string(99) == "unknown status"


def test_create_rejects_bad_arguments_without_gpu():
    lib = binding.library()
    assert lib.gemm_create(None, 0) == binding.GEMM_ERR_INVALID_ARG
    import ctypes
    h = ctypes.c_void_p()
    assert lib.gemm_create(ctypes.byref(h), -1) == binding.GEMM_ERR_INVALID_ARG
    assert lib.gemm_destroy(None) == binding.GEMM_OK
    assert lib.gemm_run(None, 1, 1, 16, 2, 1, 1, 1, 16, 16, 16, 16, 16, 4, None) == binding.GEMM_ERR_INVALID_ARG


def test_splitk_plan():
    """Split count, clamping and workspace size as the header states."""
    OK = binding.GEMM_OK
    # a partial wave: 1024 x 1024 at 128x128 is 64 tiles for 256 CUs
    rc, info = q(M=1024, N=1024, K=8192, tile="128x128", splits=0)
    assert rc == OK and info["c_tiles"] == 64 and info["splits"] == 4 and info["grid"] == 256
    assert info["workspace_bytes"] == 65536 + 64 * 4 * 128 * 128 * 4
    # explicit counts; clamped to K / (the class's largest K-tile) and to 64
    rc, info = q(M=1024, N=1024, K=8192, tile="128x128", splits=3)
    assert rc == OK and info["splits"] == 3 and info["grid"] == 192
    rc, info = q(M=1024, N=1024, K=200, tile="128x128", splits=8)     # bf16 BK 64: 3 whole units
    assert rc == OK and info["splits"] == 3
    rc, info = q(M=1024, N=1024, K=56, tile="128x128", splits=8)      # less than one unit: no split
    assert rc == OK and info["splits"] == 1 and info["workspace_bytes"] == 0
    rc, info = q(M=64, N=64, K=1 << 20, tile="32x64", splits=100)
    assert rc == OK and info["splits"] == 64
    # enough tiles already: auto takes no split; splits = 1 is gemm_run's plan
    rc, info = q(splits=0)
    assert rc == OK and info["splits"] == 1 and info["workspace_bytes"] == 0
    assert q(splits=1)[1] == q()[1]
    # the 256x256 tiles loop over work items when there are more than CUs
    rc, info = q(M=2048, N=2048, K=8192, tile="256x256", splits=8)
    assert rc == OK and info["c_tiles"] == 64 and info["splits"] == 8 and info["grid"] == 256
    # stages and variants share the split's K units (largest K-tile of the class)
    for stages in (1, 2, 3, 4):
        for variant in ("reg", "direct"):
            rc, info = q(M=512, N=512, K=8192, tile="256x256", stages=stages, variant=variant, splits=0)
            assert rc == OK and info["splits"] == 8          # the automatic choice stops at 8
            rc, info = q(M=512, N=512, K=8192, tile="256x256", stages=stages, variant=variant, splits=64)
            assert rc == OK and info["splits"] == 64
    # the automatic choice leaves at least two K units per split
    rc, info = q(M=256, N=256, K=5 * 64, tile="256x256", splits=0)
    assert rc == OK and info["splits"] == 2


def test_splitk_arguments():
    E, A, U = binding.GEMM_ERR_INVALID_ARG, binding.GEMM_ERR_ALIGNMENT, binding.GEMM_ERR_UNSUPPORTED
    assert q(splits=-1)[0] == E
    # more than 16384 C tiles cannot take a split
    assert q(M=8192, N=8192 * 4, K=8192, tile="32x64", splits=2)[0] == U
    assert q(M=8192, N=8192 * 4, K=8192, tile="32x64", splits=1)[0] == binding.GEMM_OK


def test_splitk_run_rejects_null_handle():
    """gemm_run_splitk checks its handle before anything else (the workspace
    checks need a device and are GPU-tested)."""
    lib = binding.library()
    rc = lib.gemm_run_splitk(None, 1024, 1024, 8192, 2, 1, 2, 1, 4, 16, 8192, 16, 8192, 16, 1024,
                             256, 1 << 30, None)
    assert rc == binding.GEMM_ERR_INVALID_ARG


def test_splitk_noalloc_rejects_null_handle():
    """gemm_run_splitk_noalloc checks its handle before anything else (its
    scratch-size check needs a handle, i.e. a device, and is GPU-tested)."""
    lib = binding.library()
    rc = lib.gemm_run_splitk_noalloc(None, 1024, 1024, 8192, 2, 1, 2, 1, 4, 16, 8192, 16, 8192, 16, 1024, None)
    assert rc == binding.GEMM_ERR_INVALID_ARG


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    assert "#define GEMM_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)" in text
    assert binding.GEMM_NOALLOC_SCRATCH_BYTES == 32 * 1024 * 1024


def test_occupancy_rejects_null_handle():
    lib = binding.library()
    out = binding.Occupancy()
    import ctypes
    assert lib.gemm_occupancy(None, 256, 256, 256, 3, 0, 2, 0, ctypes.byref(out)) == binding.GEMM_ERR_INVALID_ARG


def qs(M=5120, N=5120, K=5120, dtype="bf16", layout="RC", stages=3, variant="direct", tile="auto", grid=0):
    return binding.gemm_query_streamk(M, N, K, dtype, layout, stages, variant, grid=grid, tile=tile, check=False)


def test_streamk_plan():
    """Stream-K rounds, grid and workspace as the header states."""
    OK = binding.GEMM_OK
    part = 256 * 256 * 4
    # 400 tiles of 256x256 on 256 workgroups: less than two rounds, all stream-K
    rc, info = qs()
    assert rc == OK and info["tile"] == binding.GEMM_TILE_256x256 and info["c_tiles"] == 400
    assert info["sk_tiles"] == 400 and info["grid"] == 256 and info["splits"] == 1
    assert info["workspace_bytes"] == 65536 + 2 * 256 * part
    # 1100 tiles (4.3 rounds): three rounds data-parallel, the rest stream-K
    rc, info = qs(M=256 * 44, N=256 * 25)
    assert rc == OK and info["c_tiles"] == 1100 and info["sk_tiles"] == 1100 - 3 * 256
    # an explicit grid; the grid is at most the number of units
    rc, info = qs(grid=100)
    assert rc == OK and info["grid"] == 100 and info["sk_tiles"] == 400 - 100 * 3
    rc, info = qs(M=256, N=256, K=3 * 64, tile="256x256", grid=50)   # one tile of three 64-wide units
    assert rc == OK and info["grid"] == 3 and info["sk_tiles"] == 1
    rc, info = qs(M=256, N=256, K=40, tile="256x256", grid=50)       # K below one unit: one unit
    assert rc == OK and info["grid"] == 1 and info["sk_tiles"] == 1
    # nothing to do: no stream-K tiles, no workspace
    rc, info = qs(M=0)
    assert rc == OK and info["sk_tiles"] == 0 and info["workspace_bytes"] == 0
    # the tile choice is gemm_run's; the same for every (stages, variant)
    for stages in (1, 2, 3, 4):
        for variant in ("reg", "direct"):
            rc, info = qs(M=1000, N=1000, K=1000, stages=stages, variant=variant)
            assert rc == OK and info["tile"] == q(M=1000, N=1000, K=1000, stages=stages, variant=variant)[1]["tile"]


def test_streamk_arguments():
    E, U = binding.GEMM_ERR_INVALID_ARG, binding.GEMM_ERR_UNSUPPORTED
    assert qs(grid=-1)[0] == E
    # more than 16384 C tiles
    assert qs(M=8192, N=8192 * 4, K=8192, tile="32x64")[0] == U
    # partial tiles past 2 GiB: 2 x 4096 x 256 KiB
    assert qs(M=256 * 64, N=256 * 64, grid=4096)[0] == U
    assert qs(M=256 * 64, N=256 * 64, grid=4000)[0] == binding.GEMM_OK
    lib = binding.library()
    rc = lib.gemm_run_streamk(None, 5120, 5120, 5120, 2, 1, 3, 1, 0, 16, 5120, 16, 5120, 16, 5120,
                              256, 1 << 30, None)
    assert rc == E


def test_run_rejects_bad_tensors_without_gpu():
    """binding.run checks its tensors before any HIP call."""
    import torch
    a = torch.zeros(4, 8, dtype=torch.bfloat16)
    b = torch.zeros(5, 8, dtype=torch.bfloat16)
    for args in ((a, b), (a, b.half()), (a.double(), b.double()), (a, b[:, :4]), (a[0], b)):
        with pytest.raises(ValueError):
            binding.run(*args)
