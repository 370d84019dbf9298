"""Thin ctypes binding of libpipegemm.so (the C ABI in include/pipegemm.h).

Argument marshalling only: every step of the GEMM runs in the HIP kernels.
The functions keep the C names; device buffers are passed as torch CUDA
tensors (their data_ptr) or plain integer addresses.  There is no fallback:
if the library is missing, loading raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpipegemm.so")

GEMM_I8, GEMM_F16, GEMM_BF16, GEMM_F32 = 0, 1, 2, 3
GEMM_LAYOUT_RR, GEMM_LAYOUT_RC = 0, 1
GEMM_VARIANT_REG, GEMM_VARIANT_DIRECT = 0, 1
GEMM_OK, GEMM_ERR_INVALID_ARG, GEMM_ERR_ALIGNMENT, GEMM_ERR_UNSUPPORTED, GEMM_ERR_HIP = 0, 1, 2, 3, 4
GEMM_ERR_SCRATCH = 5
GEMM_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
GEMM_TILE_AUTO, GEMM_TILE_256x256, GEMM_TILE_128x128, GEMM_TILE_32x64, GEMM_TILE_256x256_W8 = -1, 0, 1, 2, 3

DTYPES = {"i8": GEMM_I8, "f16": GEMM_F16, "bf16": GEMM_BF16, "f32": GEMM_F32}
LAYOUTS = {"RR": GEMM_LAYOUT_RR, "RC": GEMM_LAYOUT_RC}
VARIANTS = {"reg": GEMM_VARIANT_REG, "direct": GEMM_VARIANT_DIRECT}
TILES = {"auto": GEMM_TILE_AUTO, "256x256": GEMM_TILE_256x256, "128x128": GEMM_TILE_128x128,
         "32x64": GEMM_TILE_32x64, "256x256w8": GEMM_TILE_256x256_W8}

# C functions exported by the library (the names include/pipegemm.h declares)
EXPORTS = ("gemm_create", "gemm_run", "gemm_destroy", "gemm_set_tile", "gemm_query",
           "gemm_run_splitk", "gemm_query_splitk", "gemm_status_string", "gemm_last_hip_error",
           "gemm_run_splitk_noalloc", "gemm_occupancy", "gemm_run_streamk", "gemm_query_streamk")


class GemmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = "%s: %s" % (where, gemm_status_string(status))
        if status == GEMM_ERR_HIP:
            msg += " (hipError %d)" % _lib().gemm_last_hip_error()
        super().__init__(msg)


class ConfigInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "tile", "block_m", "block_n", "block_k", "waves_m", "waves_n", "threads", "lds_slots",
        "reg_sets", "tiles_in_flight", "lds_bytes", "loads_per_tile")] + [
        ("grid", ctypes.c_int64), ("k_tiles", ctypes.c_int64), ("k_tail", ctypes.c_int32),
        ("c_tiles", ctypes.c_int32), ("splits", ctypes.c_int32), ("mfma_block", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64), ("waves_k", ctypes.c_int32), ("sk_tiles", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class Occupancy(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "blocks_per_cu", "waves_per_cu", "num_regs", "lds_bytes", "scratch_bytes", "threads")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpipegemm.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.gemm_create.argtypes = [ctypes.POINTER(vp), ci]
        lib.gemm_create.restype = ci
        lib.gemm_run.argtypes = [vp, i64, i64, i64, ci, ci, ci, ci, vp, i64, vp, i64, vp, i64, vp]
        lib.gemm_run.restype = ci
        lib.gemm_destroy.argtypes = [vp]
        lib.gemm_destroy.restype = ci
        lib.gemm_set_tile.argtypes = [vp, ci]
        lib.gemm_set_tile.restype = ci
        lib.gemm_query.argtypes = [i64, i64, i64, ci, ci, ci, ci, ci, vp, i64, vp, i64, vp, i64,
                                   ctypes.POINTER(ConfigInfo)]
        lib.gemm_query.restype = ci
        lib.gemm_run_splitk.argtypes = [vp, i64, i64, i64, ci, ci, ci, ci, ci, vp, i64, vp, i64, vp, i64,
                                        vp, i64, vp]
        lib.gemm_run_splitk.restype = ci
        lib.gemm_run_streamk.argtypes = [vp, i64, i64, i64, ci, ci, ci, ci, ci, vp, i64, vp, i64, vp, i64,
                                         vp, i64, vp]
        lib.gemm_run_streamk.restype = ci
        lib.gemm_query_streamk.argtypes = [i64, i64, i64, ci, ci, ci, ci, ci, ci, vp, i64, vp, i64, vp, i64,
                                           ctypes.POINTER(ConfigInfo)]
        lib.gemm_query_streamk.restype = ci
        lib.gemm_run_splitk_noalloc.argtypes = [vp, i64, i64, i64, ci, ci, ci, ci, ci, vp, i64, vp, i64, vp,
                                                i64, vp]
        lib.gemm_run_splitk_noalloc.restype = ci
        lib.gemm_occupancy.argtypes = [vp, i64, i64, i64, ci, ci, ci, ci, ctypes.POINTER(Occupancy)]
        lib.gemm_occupancy.restype = ci
        lib.gemm_query_splitk.argtypes = [i64, i64, i64, ci, ci, ci, ci, ci, ci, vp, i64, vp, i64, vp, i64,
                                          ctypes.POINTER(ConfigInfo)]
        lib.gemm_query_splitk.restype = ci
        lib.gemm_status_string.argtypes = [ci]
        lib.gemm_status_string.restype = ctypes.c_char_p
        lib.gemm_last_hip_error.argtypes = []
        lib.gemm_last_hip_error.restype = ci
        _L = lib
    return _L


def library():
    """The loaded ctypes library (loads it on first call)."""
    return _lib()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _enum(x, table):
    return table[x] if isinstance(x, str) else int(x)


def gemm_status_string(status):
    return _lib().gemm_status_string(int(status)).decode()


def gemm_create(device=0):
    h = ctypes.c_void_p()
    rc = _lib().gemm_create(ctypes.byref(h), int(device))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_create")
    return h


def gemm_destroy(h):
    _lib().gemm_destroy(h)


def gemm_set_tile(h, tile):
    rc = _lib().gemm_set_tile(h, _enum(tile, TILES))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_set_tile")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def gemm_run(h, M, N, K, dtype, layout, stages, variant, A, lda, B, ldb, C, ldc, stream=None,
             check=True):
    """Enqueue C = A * B; returns the status (raises on error when check)."""
    rc = _lib().gemm_run(h, M, N, K, _enum(dtype, DTYPES), _enum(layout, LAYOUTS), int(stages),
                         _enum(variant, VARIANTS), _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                         _stream(stream))
    if check and rc != GEMM_OK:
        raise GemmError(rc, "gemm_run")
    return rc


def gemm_run_splitk(h, M, N, K, dtype, layout, stages, variant, splits, A, lda, B, ldb, C, ldc,
                    workspace, workspace_bytes, stream=None, check=True):
    """Enqueue C = A * B with K split over `splits` workgroups per C tile."""
    rc = _lib().gemm_run_splitk(h, M, N, K, _enum(dtype, DTYPES), _enum(layout, LAYOUTS), int(stages),
                                _enum(variant, VARIANTS), int(splits), _ptr(A), lda, _ptr(B), ldb,
                                _ptr(C), ldc, _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and rc != GEMM_OK:
        raise GemmError(rc, "gemm_run_splitk")
    return rc


def gemm_run_streamk(h, M, N, K, dtype, layout, stages, variant, grid, A, lda, B, ldb, C, ldc,
                     workspace, workspace_bytes, stream=None, check=True):
    """Enqueue C = A * B with the tiles shared out stream-K over `grid`
    workgroups (0: one per compute unit)."""
    rc = _lib().gemm_run_streamk(h, M, N, K, _enum(dtype, DTYPES), _enum(layout, LAYOUTS), int(stages),
                                 _enum(variant, VARIANTS), int(grid), _ptr(A), lda, _ptr(B), ldb,
                                 _ptr(C), ldc, _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and rc != GEMM_OK:
        raise GemmError(rc, "gemm_run_streamk")
    return rc


def gemm_run_splitk_noalloc(h, M, N, K, dtype, layout, stages, variant, splits, A, lda, B, ldb, C, ldc,
                            stream=None, check=True):
    """Enqueue C = A * B with K split over `splits` workgroups per C tile,
    using the library's static scratch buffer (no workspace argument)."""
    rc = _lib().gemm_run_splitk_noalloc(h, M, N, K, _enum(dtype, DTYPES), _enum(layout, LAYOUTS), int(stages),
                                        _enum(variant, VARIANTS), int(splits), _ptr(A), lda, _ptr(B), ldb,
                                        _ptr(C), ldc, _stream(stream))
    if check and rc != GEMM_OK:
        raise GemmError(rc, "gemm_run_splitk_noalloc")
    return rc


def gemm_occupancy(h, M, N, K, dtype, layout, stages, variant):
    """Resources and occupancy of the instance gemm_run would launch (a dict)."""
    out = Occupancy()
    rc = _lib().gemm_occupancy(h, M, N, K, _enum(dtype, DTYPES), _enum(layout, LAYOUTS), int(stages),
                               _enum(variant, VARIANTS), ctypes.byref(out))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_occupancy")
    return out.as_dict()


def gemm_query(M, N, K, dtype, layout, stages, variant, tile="auto", A=0, lda=None, B=0,
               ldb=None, C=0, ldc=None, check=True, splits=1):
    """The configuration gemm_run (gemm_run_splitk with `splits`) would use
    (no HIP call).  Returns (status, dict)."""
    layout_v = _enum(layout, LAYOUTS)
    lda = K if lda is None else lda
    ldb = (N if layout_v == GEMM_LAYOUT_RR else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    info = ConfigInfo()
    rc = _lib().gemm_query_splitk(M, N, K, _enum(dtype, DTYPES), layout_v, int(stages),
                                  _enum(variant, VARIANTS), _enum(tile, TILES), int(splits), A, lda, B,
                                  ldb, C, ldc, ctypes.byref(info))
    if check and rc != GEMM_OK:
        raise GemmError(rc, "gemm_query")
    return rc, info.as_dict()


def gemm_query_streamk(M, N, K, dtype, layout, stages, variant, grid=0, tile="auto", A=0, lda=None, B=0,
                       ldb=None, C=0, ldc=None, check=True):
    """The configuration gemm_run_streamk would use (no HIP call).  Returns
    (status, dict)."""
    layout_v = _enum(layout, LAYOUTS)
    lda = K if lda is None else lda
    ldb = (N if layout_v == GEMM_LAYOUT_RR else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    info = ConfigInfo()
    rc = _lib().gemm_query_streamk(M, N, K, _enum(dtype, DTYPES), layout_v, int(stages),
                                   _enum(variant, VARIANTS), _enum(tile, TILES), int(grid), A, lda, B,
                                   ldb, C, ldc, ctypes.byref(info))
    if check and rc != GEMM_OK:
        raise GemmError(rc, "gemm_query_streamk")
    return rc, info.as_dict()


_HANDLES = {}   # device index -> Gemm, for run()


def run(a, b, *, layout="RC", stages=2, variant="direct", out=None, stream=None):
    """C = A * B on torch CUDA tensors through gemm_run.

    A is M x K row-major; B is K x N row-major for layout "RR", or its N x K
    transpose (B column-major) for "RC".  The element type is A's (int8,
    float16, bfloat16 or float32; B must match); C is int32 for int8 and A's
    type otherwise.  `out` (M x N, unit stride along the last axis) is
    written in place, else a new tensor is allocated.  The call is enqueued
    on `stream` (the current stream of A's device by default) and C is
    returned.  Argument errors raise ValueError before any HIP call."""
    import torch
    names = {torch.int8: "i8", torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}
    outs = {"i8": torch.int32, "f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    if not (isinstance(a, torch.Tensor) and isinstance(b, torch.Tensor)) or a.dim() != 2 or b.dim() != 2:
        raise ValueError("A and B must be 2-D torch tensors")
    if a.dtype not in names or b.dtype != a.dtype:
        raise ValueError("A and B must share one of int8, float16, bfloat16, float32 (got %s, %s)"
                         % (a.dtype, b.dtype))
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("A and B must be CUDA tensors on one device")
    dtype = names[a.dtype]
    M, K = a.shape
    if _enum(layout, LAYOUTS) == GEMM_LAYOUT_RR:
        Kb, N = b.shape
    else:
        N, Kb = b.shape
    if Kb != K:
        raise ValueError("inner dimensions differ: A has K = %d, B has %d" % (K, Kb))
    if out is None:
        out = torch.empty((M, N), dtype=outs[dtype], device=a.device)
    elif (not isinstance(out, torch.Tensor) or out.dtype != outs[dtype] or tuple(out.shape) != (M, N)
          or out.device != a.device):
        raise ValueError("out must be an M x N %s tensor on A's device" % outs[dtype])
    dev = a.device.index if a.device.index is not None else torch.cuda.current_device()
    g = _HANDLES.get(dev)
    if g is None:
        g = _HANDLES[dev] = Gemm(dev)
    g.run(a, b, out, dtype, layout, stages, variant,
          stream if stream is not None else torch.cuda.current_stream(a.device))
    return out


class Gemm:
    """Owns a handle; ``run`` takes torch CUDA tensors in the ABI's storage:
    A (M x K row-major), B (K x N row-major for RR, its N x K transpose for
    RC), C (M x N row-major)."""

    def __init__(self, device=0):
        self.h = gemm_create(device)
        self.device = device
        self.tile = "auto"
        self._ws = None   # split-K workspace: zeroed once, left zeroed by every call

    def workspace(self, nbytes):
        """A device buffer of at least nbytes for gemm_run_splitk / gemm_run_streamk (grown,
        zeroed, on demand)."""
        import torch
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device="cuda:%d" % self.device)
        return self._ws

    def close(self):
        if self.h is not None:
            gemm_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_tile(self, tile):
        gemm_set_tile(self.h, tile)
        self.tile = tile

    def run(self, a, b, c, dtype, layout, stages, variant, stream=None, splits=1):
        M, K = a.shape
        N = b.shape[1] if _enum(layout, LAYOUTS) == GEMM_LAYOUT_RR else b.shape[0]
        for t in (a, b, c):
            if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
                raise ValueError("operands must be 2-D with unit stride along the last axis")
        if splits == 1:
            return gemm_run(self.h, M, N, K, dtype, layout, stages, variant,
                            a, a.stride(0), b, b.stride(0), c, c.stride(0), stream)
        return self.run_splitk(M, N, K, dtype, layout, stages, variant, splits, a, a.stride(0), b,
                               b.stride(0), c, c.stride(0), stream)

    def run_splitk(self, M, N, K, dtype, layout, stages, variant, splits, A, lda, B, ldb, C, ldc,
                   stream=None, check=True):
        """gemm_run_splitk with this handle's tile and workspace."""
        _, info = gemm_query(M, N, K, dtype, layout, stages, variant, tile=self.tile, lda=lda, ldb=ldb,
                             ldc=ldc, splits=splits, check=False)
        ws = self.workspace(info["workspace_bytes"]) if info["workspace_bytes"] > 0 else None
        return gemm_run_splitk(self.h, M, N, K, dtype, layout, stages, variant, splits, A, lda, B, ldb,
                               C, ldc, ws, ws.numel() if ws is not None else 0, stream, check)

    def run_streamk(self, M, N, K, dtype, layout, stages, variant, grid, A, lda, B, ldb, C, ldc,
                    stream=None, check=True):
        """gemm_run_streamk with this handle's tile and workspace."""
        _, info = gemm_query_streamk(M, N, K, dtype, layout, stages, variant, grid=grid, tile=self.tile,
                                     lda=lda, ldb=ldb, ldc=ldc, check=False)
        ws = self.workspace(info["workspace_bytes"]) if info["workspace_bytes"] > 0 else None
        return gemm_run_streamk(self.h, M, N, K, dtype, layout, stages, variant, grid, A, lda, B, ldb, C, ldc,
                                ws, 0 if ws is None else ws.numel(), stream, check)
