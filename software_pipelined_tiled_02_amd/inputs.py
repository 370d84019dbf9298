"""Seeded synthetic GEMM operands.

This module holds no matrix-product arithmetic: it only draws random numbers,
casts them to the element type and hands them out in the storage each side
needs (torch CPU tensors for the HIP path, numpy arrays in the oracle's
encodings for the oracle).  Both sides consume the *same* cast arrays, so the
choice of random generator never affects parity.

Conventions (the pages leave "from seed" open; this is the reading used):
  - A draws from ``torch.Generator().manual_seed(seed)``, B from ``seed + 1``.
  - "uniform"  : 2 * U[0,1) - 1 in float32, then cast (entries in [-1, 1)).
  - "normal"   : N(0, 1) in float32, times ``scale``, then cast.
  - "int"      : uniform integers in [-128, 127] (int8 only).
A is row-major M x K.  B is row-major K x N for layout "RR" and, for layout
"RC" (B column-major, K contiguous), stored as its N x K transpose.
"""
import numpy as np
import torch

TORCH_DTYPES = {"i8": torch.int8, "f16": torch.float16, "bf16": torch.bfloat16,
                "f32": torch.float32}
OUT_TORCH_DTYPES = {"i8": torch.int32, "f16": torch.float16, "bf16": torch.bfloat16,
                    "f32": torch.float32}


def _draw(shape, dist, dtype, gen, scale):
    if dist == "int":
        if dtype != "i8":
            raise ValueError("integer draws are for int8 only")
        return torch.randint(-128, 128, shape, generator=gen, dtype=torch.int16).to(torch.int8)
    if dist == "uniform":
        x = 2.0 * torch.rand(shape, generator=gen, dtype=torch.float32) - 1.0
    elif dist == "normal":
        x = torch.randn(shape, generator=gen, dtype=torch.float32)
    else:
        raise ValueError("unknown distribution %r" % dist)
    if scale != 1.0:
        x = x * scale
    if dtype == "i8":
        raise ValueError("int8 operands use dist='int'")
    return x.to(TORCH_DTYPES[dtype])


def make_operands(M, N, K, dtype, layout, dist, seed=0, scale=1.0):
    """Return (A, B) as contiguous torch CPU tensors in the storage above."""
    ga = torch.Generator().manual_seed(seed)
    gb = torch.Generator().manual_seed(seed + 1)
    a = _draw((M, K), dist, dtype, ga, scale)
    b_shape = (K, N) if layout == "RR" else (N, K)
    b = _draw(b_shape, dist, dtype, gb, scale)
    return a.contiguous(), b.contiguous()


def to_oracle(t, dtype):
    """A torch CPU tensor as a numpy array in the oracle's element encoding."""
    t = t.contiguous()
    if dtype in ("f16", "bf16"):
        return t.view(torch.int16).numpy().view(np.uint16)
    if dtype == "i8":
        return t.numpy().view(np.int8)
    return t.numpy().astype(np.float32, copy=False)


def from_torch_out(c, dtype):
    """A result tensor (any device) as a numpy array: int32 or float64."""
    c = c.detach().cpu()
    if dtype == "i8":
        return c.numpy().astype(np.int32, copy=False)
    return c.float().numpy().astype(np.float64)
