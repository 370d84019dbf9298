#!/usr/bin/env python3
"""Benchmark of the pipelined tiled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rounds R] [--workload NAME]
                    [--tile T] [--splits P]

A step is one C = A * B launch (the whole K-loop pipeline: prologue, main
loop, drain, epilogue) over one synthetic input set.  After half a second
of untimed launches that lets the GPU clocks settle, every (stages,
variant) pair of the chosen workload is timed, in R rounds over all pairs:
each time W untimed warm-up steps, then exactly K steps launched back to
back between two HIP events recorded on the stream the kernel is launched
on (synchronised on both sides); the launch duration is that interval over
K, and a pair reports its median round (all rounds are in "rounds_us").  A
last pass of K launches per pair, each between its own events, gives the
spread (per_launch_* in "sweep").
Inputs rotate over enough copies that the footprint exceeds 512 MiB, so
the 256 MB Infinity Cache cannot hold them.
The headline is the fastest pair; all pairs are in "sweep".

Prints one JSON line.  `value` is TOP/s (int8) or TFLOP/s (fp) counting
2*M*N*K operations (the convention of the pipelining study's benchmark
table), or GB/s of algorithmic bytes for the memory-bound skinny shape.
`roofline` compares the headline kernel with MI355X's published peak for
its dtype; `cpu_baseline` is the CPU oracle timed on a bounded sample on
this host's cores.
"""
import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# name: (M, N, K, dtype, layout, dist, scale, bound, description)
WORKLOADS = {
    "int8_4096": (4096, 4096, 4096, "i8", "RC", "int", 1.0, "mfma",
                  "int8 IGEMM M=N=K=4096, A row-major, B column-major, int32 out"),
    "fp16_4096": (4096, 4096, 4096, "f16", "RC", "normal", 1.0 / 64.0, "mfma",
                  "fp16 GEMM M=N=K=4096, N(0,1)/sqrt(K) entries, fp32 accumulate, fp16 out"),
    "bf16_skinny": (8192, 64, 8192, "bf16", "RC", "normal", 1.0, "hbm",
                    "bf16 GEMM M=8192 N=64 K=8192, fp32 accumulate, bf16 out"),
    "bf16_8192x8200": (8192, 8192, 8200, "bf16", "RC", "uniform", 1.0, "mfma",
                       "bf16 GEMM M=N=8192 K=8200 (ragged last K-tile), fp32 accumulate, bf16 out"),
    "fp32_256": (256, 256, 256, "f32", "RR", "uniform", 1.0, "mfma",
                 "fp32 GEMM M=N=K=256, A and B row-major"),
    "fp16_4096_rr": (4096, 4096, 4096, "f16", "RR", "normal", 1.0 / 64.0, "mfma",
                     "fp16 GEMM M=N=K=4096, A and B row-major (B read with transposing LDS reads)"),
    "int8_4096_rr": (4096, 4096, 4096, "i8", "RR", "int", 1.0, "mfma",
                     "int8 IGEMM M=N=K=4096, A and B row-major (B read with transposing LDS reads)"),
    "bf16_1024x1024x8192": (1024, 1024, 8192, "bf16", "RC", "uniform", 1.0, "mfma",
                            "bf16 GEMM M=N=1024 K=8192 (few C tiles, long K), fp32 accumulate, bf16 out"),
    "bf16_1024x8192x8200": (1024, 8192, 8200, "bf16", "RC", "uniform", 1.0, "mfma",
                            "bf16 GEMM M=1024 N=8192 K=8200 (one GPU's share of M=N=8192 K=8200 "
                            "split 8 ways along M), fp32 accumulate, bf16 out"),
}
DEFAULT_WORKLOAD = "int8_4096"

# MI355X published dense peaks (per GPU)
PEAK = {"i8": 5033.2, "f16": 2516.6, "bf16": 2516.6, "f32": 157.3}   # TOP/s, TFLOP/s
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 512 * 2 ** 20


def flops(M, N, K):
    """Operations of C = A * B: one multiply and one add per (i, j, k)."""
    return 2.0 * M * N * K


def kernel_source_hash():
    """Hash of the library's sources with comments and white space removed,
    so that only a change of code marks measured counters as stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "software_pipelined_tiled_02_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".h", ".hip")) and not name.endswith("_probe.hip"):   # probes are no GEMM source
            text = open(os.path.join(csrc, name), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(name.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload, stages, variant):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    key = "hbm_bytes_per_launch_S%d_%s" % (stages, variant)
    return float(vals[key]) if key in vals else None


def measured_ceiling(dtype, bound, block=32):
    """The chip's attainable rate for this dtype (MFMA loop of the kernel's
    block shape, fed from LDS with random data) or for HBM (streaming read),
    from the committed output of ceiling_probe; None if absent."""
    path = os.path.join(ROOT, "profiles", "ceilings.txt")
    if not os.path.exists(path):
        return None
    prefix = "mfma16_" if block == 16 else "mfma_"
    key = "hbm_read" if bound == "hbm" else prefix + {"i8": "int8", "f16": "fp16", "bf16": "bf16", "f32": "fp32"}[dtype]
    for line in open(path):
        if line.startswith(key + ":"):
            return float(line.split(":", 1)[1].split()[0])
    return None


def host_cpu():
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(M, N, K, dtype, layout, dist, scale, target_s):
    """The oracle, untuned, on a bounded row sample of the same workload."""
    import oracle
    from software_pipelined_tiled_02_amd import inputs

    a, b = inputs.make_operands(M, N, K, dtype, layout, dist, seed=0, scale=scale)
    an, bn = inputs.to_oracle(a, dtype), inputs.to_oracle(b, dtype)
    orc = oracle.default()
    rows = max(1, min(M, 8))
    t0 = time.perf_counter()
    orc.gemm(an[:rows], bn, dtype, layout)
    t1 = time.perf_counter() - t0
    rows = int(min(M, max(rows, rows * target_s / max(t1, 1e-6))))
    t0 = time.perf_counter()
    orc.gemm(an[:rows], bn, dtype, layout)
    el = time.perf_counter() - t0
    return {"value": round(flops(rows, N, K) / el / 1e12, 6),
            "unit": "TOP/s" if dtype == "i8" else "TFLOP/s",
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": "first %d of %d rows of C (%dx%dx%d), %.1f s wall, host %s" % (
                rows, M, rows, N, K, el, host_cpu())}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--rounds", type=int, default=3, help="rounds over all pairs; each pair reports its median")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--pairs", default="all", help="comma list like 3:direct,2:reg, or all")
    ap.add_argument("--tile", default="auto", help="tile class: auto, 256x256, 256x256w8, 128x128, 32x64")
    ap.add_argument("--splits", type=int, default=1,
                    help="K splits per C tile (gemm_run_splitk); 0 = the library's choice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this GEMM is measured on a single MI355X "
              "(--gpus %d requested); multi-GPU runs are not part of this build." % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from software_pipelined_tiled_02_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    M, N, K, dtype, layout, dist, scale, bound, desc = WORKLOADS[args.workload]
    if args.pairs == "all":
        pairs = [(s, v) for s in (1, 2, 3, 4) for v in ("reg", "direct")]
    else:
        pairs = [(int(p.split(":")[0]), p.split(":")[1]) for p in args.pairs.split(",")]

    g = binding.Gemm(0)
    g.set_tile(args.tile)
    a, b = inputs.make_operands(M, N, K, dtype, layout, dist, seed=0, scale=scale)
    a, b = a.cuda(), b.cuda()
    out_dt = inputs.OUT_TORCH_DTYPES[dtype]
    c_bytes = M * N * torch.tensor([], dtype=out_dt).element_size()
    set_bytes = a.numel() * a.element_size() + b.numel() * b.element_size() + c_bytes
    nrot = max(1, -(-ROTATE_BYTES // set_bytes))
    sets = [(a if i == 0 else a.clone(), b if i == 0 else b.clone(),
             torch.empty((M, N), dtype=out_dt, device="cuda")) for i in range(nrot)]
    ldb = N if layout == "RR" else K
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    if args.splits != 1:
        # the split-K workspace, allocated (zeroed) once, before anything is timed
        for s, v in pairs:
            _, qi = binding.gemm_query(M, N, K, dtype, layout, s, v, tile=args.tile, splits=args.splits)
            g.workspace(qi["workspace_bytes"])
    ws = g.workspace(1) if args.splits != 1 else None

    def run_one(aa, bb, cc, s, v):
        if args.splits == 1:
            binding.gemm_run(g.h, M, N, K, dtype, layout, s, v, aa, K, bb, ldb, cc, N, sh)
        else:
            binding.gemm_run_splitk(g.h, M, N, K, dtype, layout, s, v, args.splits, aa, K, bb, ldb, cc, N,
                                    ws, ws.numel(), sh)

    def launch(i, s, v):
        run_one(*sets[i % nrot], s, v)

    ops = flops(M, N, K)
    algo_bytes = set_bytes
    # Bring the GPU out of its idle clock state before anything is timed:
    # run the first pair for about half a second (a fixed count of short
    # launches is not enough for the clocks to settle).
    t_end = time.perf_counter() + 0.5
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(10):
            launch(i, *pairs[0])
            i += 1
        torch.cuda.synchronize()
    # The sweep runs in `rounds` rounds, each timing every pair once; a pair
    # is reported by its median round.  (Measured in one sweep, the same
    # kernel came out 20-30% slower when it happened to be timed third, a
    # window in which the chip's clock drops; rounds spread every pair over
    # the run instead of tying it to one moment.)
    rounds = {p: [] for p in pairs}
    first_c = None          # C of the first pair: every pair must reproduce it bit for bit
    identical = True
    for rnd in range(args.rounds):
        for s, v in pairs:
            for i in range(args.warmup):
                launch(i, s, v)
            torch.cuda.synchronize()
            # The timed region: K launches back to back between two events on
            # the launch stream, synchronised on both sides.
            t_start = torch.cuda.Event(enable_timing=True)
            t_end = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t_start.record(stream)
            for i in range(args.steps):
                launch(i, s, v)
            t_end.record(stream)
            torch.cuda.synchronize()
            rounds[(s, v)].append(t_start.elapsed_time(t_end) / args.steps)   # ms per launch
            if rnd == 0:
                c0 = sets[0][2].view(torch.uint8)
                if first_c is None:
                    first_c = c0.clone()
                elif not torch.equal(c0, first_c):
                    identical = False
                    print("# S=%d %s: C differs bitwise from the first pair" % (s, v), file=sys.stderr, flush=True)
    results = {}
    for s, v in pairs:
        rs = rounds[(s, v)]
        mean = sorted(rs)[len(rs) // 2]                            # median round, ms per launch
        # Spread (informational): K launches, each between its own pair of
        # events (which adds the event records' gaps to each).
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for i in range(args.steps):
            ev[i][0].record(stream)
            launch(i, s, v)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        per = sorted(e0.elapsed_time(e1) for e0, e1 in ev)       # ms per launch
        results[(s, v)] = {
            "mean_us": round(mean * 1e3, 2), "median_us": round(per[len(per) // 2] * 1e3, 2),
            "min_us": round(per[0] * 1e3, 2), "max_us": round(per[-1] * 1e3, 2),
            "rounds_us": [round(x * 1e3, 2) for x in rs],
            "ms_per_step": mean,
            "tops": ops / (mean * 1e-3) / 1e12, "gbs": algo_bytes / (mean * 1e-3) / 1e9,
        }
        print("# %-14s S=%d %-6s median round %8.2f us  %8.1f %s  %7.1f GB/s  rounds %s" % (
            args.workload, s, v, mean * 1e3, results[(s, v)]["tops"],
            "TOP/s" if dtype == "i8" else "TFLOP/s", results[(s, v)]["gbs"],
            " ".join("%.1f" % (x * 1e3) for x in rs)), file=sys.stderr, flush=True)

    best = min(results, key=lambda p: results[p]["mean_us"])
    r = results[best]
    _, info = binding.gemm_query(M, N, K, dtype, layout, best[0], best[1], tile=args.tile, splits=args.splits)
    unit = "TOP/s" if dtype == "i8" else "TFLOP/s"
    if bound == "hbm":
        value, vunit = r["gbs"], "GB/s"
        roof = {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(r["gbs"] / HBM_PEAK_GBS, 4)}
    else:
        value, vunit = r["tops"], unit
        roof = {"bound": "mfma", "achieved": round(r["tops"], 1), "peak": PEAK[dtype], "unit": unit,
                "frac": round(r["tops"] / PEAK[dtype], 4)}
    roof["traffic"] = read_traffic(args.workload, best[0], best[1])
    ceil = measured_ceiling(dtype, bound, info["mfma_block"])
    if ceil:
        roof["measured_ceiling"] = {"value": ceil, "unit": roof["unit"], "frac": round(roof["achieved"] / ceil, 4),
                                    "source": "profiles/ceilings.txt (ceiling_probe: %s fed from LDS with random "
                                              "data / HBM streaming read)" % (
                                                  "%dx%d MFMA blocks" % (info["mfma_block"], info["mfma_block"]))}
    hot = None
    if bound == "hbm":
        # The same buffers every launch: A fits in the Infinity Cache, so this
        # is a cache-resident figure, reported beside (never as) the value.
        for _ in range(args.warmup):
            run_one(a, b, sets[0][2], best[0], best[1])
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(args.steps):
            run_one(a, b, sets[0][2], best[0], best[1])
        t1.record(stream)
        torch.cuda.synchronize()
        hot_ms = t0.elapsed_time(t1) / args.steps
        hot = {"us": round(hot_ms * 1e3, 2), "GB/s": round(algo_bytes / (hot_ms * 1e-3) / 1e9, 1),
               "note": "same A, B, C every launch (Infinity-Cache resident), not the headline"}

    line = {
        "metric": "GEMM TFLOP/s (int8 TOP/s) and % of MFMA peak per stage count/variant, 1 GPU",
        "value": round(value, 2), "unit": vunit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"i8": "int8", "f16": "fp16", "bf16": "bf16", "f32": "fp32"}[dtype],
        "data": "synthetic (seeded), inputs resident in HBM, rotated over %d sets (%.0f MiB)" % (
            nrot, nrot * set_bytes / 2 ** 20),
        "config": {"workload": desc, "M": M, "N": N, "K": K, "layout": layout,
                   "stages": best[0], "variant": best[1],
                   "tile": "%dx%dx%d" % (info["block_m"], info["block_n"], info["block_k"]),
                   "lds_bytes": info["lds_bytes"], "grid": info["grid"], "splits": info["splits"],
                   "mfma_block": info["mfma_block"]},
        "roofline": roof,
        "pairs_bit_identical": identical,
        "rounds": args.rounds,
        "sweep": {"S%d_%s" % p: {"us": q["mean_us"], "rounds_us": q["rounds_us"],
                                 "per_launch_median_us": q["median_us"],
                                 "per_launch_min_us": q["min_us"], "per_launch_max_us": q["max_us"],
                                 unit if bound != "hbm" else "GB/s":
                                     round(q["tops"] if bound != "hbm" else q["gbs"], 2),
                                 "frac_peak": round(q["tops"] / PEAK[dtype], 4) if bound != "hbm"
                                 else round(q["gbs"] / HBM_PEAK_GBS, 4)}
                  for p, q in results.items()},
    }
    if hot is not None:
        line["hot"] = hot
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(M, N, K, dtype, layout, dist, scale, args.cpu_seconds)
    g.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
