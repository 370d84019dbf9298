"""A plain device-to-device copy of known size, for calibrating HBM byte
counters: run it under `rocprofv3 --pmc FETCH_SIZE` (then WRITE_SIZE) and
divide the bytes it must move (printed below) by what the counter reports
per dispatch; the same factor then converts the GEMM kernels' counter
readings into HBM bytes.

    python -m software_pipelined_tiled_02_amd.hbm_copy_probe [--mib 1024] [--reps 3]
"""
import argparse

import torch


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    a = ap.parse_args()
    n = a.mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copy probe: %d dispatches, each reads %d bytes and writes %d bytes"
          % (a.reps, n * 4, n * 4), flush=True)


if __name__ == "__main__":
    main()
