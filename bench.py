#!/usr/bin/env python3
"""Benchmark of the pipelined tiled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rounds R] [--workload NAME|all]
                    [--tile T] [--splits P]

By default (--workload all) the five benchmark workloads are measured in
one run -- fp32 256^3 (layout RR), int8 4096^3, fp16 4096^3, the skinny
bf16 8192x64x8192 and bf16 8192^2 x 8200 -- and the headline `value` is the
int8 4096^3 one; every workload's figures are under "configs".

A step is one C = A * B launch (the whole K-loop pipeline: prologue, main
loop, drain, epilogue) over one synthetic input set.  After half a second
of untimed launches that lets the GPU clocks settle, every (stages,
variant) pair of a workload is timed, in R rounds over all pairs:
each time W untimed warm-up steps, then exactly K steps launched back to
back between two HIP events recorded on the stream the kernel is launched
on (synchronised on both sides); the launch duration is that interval over
K, and a pair reports its median round (all rounds are in "rounds_us").  A
last pass of K launches per pair, each between its own events, gives the
spread (per_launch_* in "sweep").
Inputs rotate over enough copies that the footprint exceeds 512 MiB, so
the 256 MB Infinity Cache cannot hold them.
A workload's figure is its fastest pair; all pairs are in "sweep" (per
workload: "pairs"), each with the occupancy of its kernel instance.
Before anything touches the GPU the chip's attainable rates are measured
by ceiling_probe (a child process), so every fraction is also given against
the ceiling of the same box.

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
import subprocess
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
    "fp32_4096_rr": (4096, 4096, 4096, "f32", "RR", "uniform", 1.0, "mfma",
                     "fp32 GEMM M=N=K=4096, A and B row-major (the fp32 comparison at a compute-bound size)"),
    "fp16_4096_rr": (4096, 4096, 4096, "f16", "RR", "normal", 1.0 / 64.0, "mfma",
                     "fp16 GEMM M=N=K=4096, A and B row-major (B read with transposing LDS reads)"),
    "int8_4096_rr": (4096, 4096, 4096, "i8", "RR", "int", 1.0, "mfma",
                     "int8 IGEMM M=N=K=4096, A and B row-major (B read with transposing LDS reads)"),
    "bf16_1024x1024x8192": (1024, 1024, 8192, "bf16", "RC", "uniform", 1.0, "mfma",
                            "bf16 GEMM M=N=1024 K=8192 (few C tiles, long K), fp32 accumulate, bf16 out"),
    "bf16_1024x8192x8200": (1024, 8192, 8200, "bf16", "RC", "uniform", 1.0, "mfma",
                            "bf16 GEMM M=1024 N=8192 K=8200 (one GPU's share of M=N=8192 K=8200 "
                            "split 8 ways along M), fp32 accumulate, bf16 out"),
    # partial last waves (tiles of 256x256 not a whole number of rounds of 256 CUs)
    "bf16_5120x5120x5128": (5120, 5120, 5128, "bf16", "RC", "uniform", 1.0, "mfma",
                            "bf16 GEMM M=N=5120 K=5128 (400 tiles of 256x256: 1.56 rounds), fp32 "
                            "accumulate, bf16 out"),
    "int8_4608x4608x4096": (4608, 4608, 4096, "i8", "RC", "int", 1.0, "mfma",
                            "int8 IGEMM M=N=4608 K=4096 (324 tiles of 256x256: 1.27 rounds), int32 out"),
    "bf16_4352x4352x4096": (4352, 4352, 4096, "bf16", "RC", "uniform", 1.0, "mfma",
                            "bf16 GEMM M=N=4352 K=4096 (289 tiles of 256x256: 1.13 rounds), fp32 "
                            "accumulate, bf16 out"),
}
# The five benchmark workloads, in the order they are measured; the first
# MFMA-bound 4096^3 one (int8) is the headline.
FIVE = ["fp32_256", "int8_4096", "fp16_4096", "bf16_skinny", "bf16_8192x8200"]
HEADLINE = "int8_4096"

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


def ceiling_key(dtype, bound, block=32):
    if bound == "hbm":
        return "hbm_read"
    prefix = "mfma16_" if block == 16 else "mfma_"
    return prefix + {"i8": "int8", "f16": "fp16", "bf16": "bf16", "f32": "fp32"}[dtype]


def parse_ceilings(text):
    """{key: value} from ceiling_probe's "key: value ..." lines."""
    out = {}
    for line in text.splitlines():
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        try:
            out[k.strip()] = float(v.split()[0])
        except (ValueError, IndexError):
            pass
    return out


def committed_ceilings():
    """The committed output of ceiling_probe (profiles/ceilings.txt), or {}."""
    path = os.path.join(ROOT, "profiles", "ceilings.txt")
    return parse_ceilings(open(path).read()) if os.path.exists(path) else {}


def measured_ceiling(dtype, bound, block=32, table=None):
    """The chip's attainable rate for this dtype (MFMA loop of the kernel's
    block shape, fed from LDS with random data) or for HBM (streaming read):
    from `table` (a same-run probe), else from the committed probe output;
    None if absent."""
    table = committed_ceilings() if table is None else table
    return table.get(ceiling_key(dtype, bound, block))


def probe_ceilings(timeout=180):
    """Run ceiling_probe as a child process (before this process touches the
    GPU); returns its table, or None if it is missing or fails."""
    exe = os.path.join(ROOT, "software_pipelined_tiled_02_amd", "ceiling_probe")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=timeout)
    except (OSError, subprocess.TimeoutExpired):
        return None
    if r.returncode != 0:
        return None
    t = parse_ceilings(r.stdout)
    return t if "mfma16_int8" in t and "hbm_read" in t else None


def kernel_resources():
    """Per-kernel register, LDS and occupancy figures the compiler reported
    when the library was built (kernel_resources.json), or {}."""
    path = os.path.join(ROOT, "software_pipelined_tiled_02_amd", "kernel_resources.json")
    return json.load(open(path)) if os.path.exists(path) else {}


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
    """The oracle, untuned, on a bounded row sample of the same workload:
    the first rows of C, as many as take about target_s seconds (sized from
    two shorter timed runs)."""
    import oracle
    from software_pipelined_tiled_02_amd import inputs

    a, b = inputs.make_operands(M, N, K, dtype, layout, dist, seed=0, scale=scale)
    an, bn = inputs.to_oracle(a, dtype), inputs.to_oracle(b, dtype)
    orc = oracle.default()

    def timed(r):
        t0 = time.perf_counter()
        orc.gemm(an[:r], bn, dtype, layout)
        return time.perf_counter() - t0

    rows = min(M, 8)
    el = timed(rows)
    while rows < M and el < 0.2 * target_s:          # grow toward a quarter of the budget
        rows = int(min(M, max(2 * rows, rows * 0.25 * target_s / max(el, 1e-6))))
        el = timed(rows)
    if rows < M and el < 0.8 * target_s:               # then the budget itself
        rows = int(min(M, rows * target_s / max(el, 1e-6)))
        el = timed(rows)
    return {"value": round(flops(rows, N, K) / el / 1e12, 6),
            "unit": "TOP/s" if dtype == "i8" else "TFLOP/s",
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": "first %d of %d rows of C (%dx%dx%d), %.1f s wall, host %s" % (
                rows, M, rows, N, K, el, host_cpu())}


def pair_key(s, v):
    return "S%d_%s" % (s, v)


def occupancy_of(g, res_table, M, N, K, dtype, layout, stages, variant, tile, info):
    """The launched instance's occupancy (runtime calculator) and the
    compiler's register split for it."""
    from software_pipelined_tiled_02_amd import binding, build
    occ = binding.gemm_occupancy(g.h, M, N, K, dtype, layout, stages, variant)
    kv = binding.VARIANTS[variant] if K % inputs_epc(dtype) == 0 or variant == "direct" else 2
    sym = build.kernel_symbol(binding.DTYPES[dtype], binding.LAYOUTS[layout], info["tile"], stages, kv)
    r = res_table.get(sym, {})
    return {"blocks_per_cu": occ["blocks_per_cu"], "waves_per_cu": occ["waves_per_cu"],
            "vgprs": r.get("vgprs"), "agprs": r.get("agprs"), "runtime_num_regs": occ["num_regs"],
            "lds_bytes": occ["lds_bytes"], "scratch_bytes_per_lane": occ["scratch_bytes"],
            "compiler_waves_per_simd": r.get("waves_per_simd")}


def inputs_epc(dtype):
    return {"i8": 16, "f16": 8, "bf16": 8, "f32": 4}[dtype]


def measure_workload(name, args, g, ceilings, res_table, pairs):
    """Time every (stages, variant) pair of one workload; returns its record
    and the inputs it drew (for the CPU baseline)."""
    import torch
    from software_pipelined_tiled_02_amd import binding, inputs

    M, N, K, dtype, layout, dist, scale, bound, desc = WORKLOADS[name]
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

    if args.splits != 1 or args.streamk:
        # the split-K / stream-K workspace, allocated (zeroed) once, before anything is timed
        for s, v in pairs:
            if args.streamk:
                _, qi = binding.gemm_query_streamk(M, N, K, dtype, layout, s, v, grid=args.sk_grid, tile=args.tile)
            else:
                _, qi = binding.gemm_query(M, N, K, dtype, layout, s, v, tile=args.tile, splits=args.splits)
            g.workspace(qi["workspace_bytes"])
    ws = g.workspace(1) if (args.splits != 1 or args.streamk) else None

    def run_one(aa, bb, cc, s, v):
        if args.streamk:
            binding.gemm_run_streamk(g.h, M, N, K, dtype, layout, s, v, args.sk_grid, aa, K, bb, ldb, cc, N,
                                     ws, ws.numel(), sh)
        elif args.splits == 1:
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
            t_stop = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t_start.record(stream)
            for i in range(args.steps):
                launch(i, s, v)
            t_stop.record(stream)
            torch.cuda.synchronize()
            rounds[(s, v)].append(t_start.elapsed_time(t_stop) / args.steps)   # ms per launch
            if rnd == 0:
                c0 = sets[0][2].view(torch.uint8)
                if first_c is None:
                    first_c = c0.clone()
                elif not torch.equal(c0, first_c):
                    identical = False
                    print("# %s S=%d %s: C differs bitwise from the first pair" % (name, s, v),
                          file=sys.stderr, flush=True)
    unit = "TOP/s" if dtype == "i8" else "TFLOP/s"
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
        if args.streamk:
            _, qi = binding.gemm_query_streamk(M, N, K, dtype, layout, s, v, grid=args.sk_grid, tile=args.tile)
        else:
            _, qi = binding.gemm_query(M, N, K, dtype, layout, s, v, tile=args.tile, splits=args.splits)
        results[(s, v)] = {
            "mean_us": round(mean * 1e3, 2), "median_us": round(per[len(per) // 2] * 1e3, 2),
            "min_us": round(per[0] * 1e3, 2), "max_us": round(per[-1] * 1e3, 2),
            "rounds_us": [round(x * 1e3, 2) for x in rs],
            "ms_per_step": mean,
            "tops": ops / (mean * 1e-3) / 1e12, "gbs": algo_bytes / (mean * 1e-3) / 1e9,
            "info": qi,
            "occupancy": occupancy_of(g, res_table, M, N, K, dtype, layout, s, v, args.tile, qi),
        }
        print("# %-14s S=%d %-6s median round %8.2f us  %8.1f %s  %7.1f GB/s  rounds %s" % (
            name, s, v, mean * 1e3, results[(s, v)]["tops"], unit, results[(s, v)]["gbs"],
            " ".join("%.1f" % (x * 1e3) for x in rs)), file=sys.stderr, flush=True)

    best = min(results, key=lambda p: results[p]["mean_us"])
    r = results[best]
    info = r["info"]
    ceil = measured_ceiling(dtype, bound, info["mfma_block"], ceilings["table"])
    if bound == "hbm":
        value, vunit, peak = r["gbs"], "GB/s", HBM_PEAK_GBS
    else:
        value, vunit, peak = r["tops"], unit, PEAK[dtype]
    roof = {"bound": bound, "achieved": round(value, 1), "peak": peak, "unit": vunit,
            "frac": round(value / peak, 4), "traffic": read_traffic(name, best[0], best[1])}
    if ceil:
        roof["measured_ceiling"] = {
            "value": ceil, "unit": vunit, "frac": round(value / ceil, 4),
            "key": ceiling_key(dtype, bound, info["mfma_block"]), "source": ceilings["source"]}
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

    def pair_record(q):
        rec = {"us": q["mean_us"], "rounds_us": q["rounds_us"], "per_launch_median_us": q["median_us"],
               "per_launch_min_us": q["min_us"], "per_launch_max_us": q["max_us"]}
        if bound == "hbm":
            rec["GB/s"] = round(q["gbs"], 2)
            rec["frac_peak"] = round(q["gbs"] / HBM_PEAK_GBS, 4)
        else:
            rec[unit] = round(q["tops"], 2)
            rec["frac_peak"] = round(q["tops"] / PEAK[dtype], 4)
        c = measured_ceiling(dtype, bound, q["info"]["mfma_block"], ceilings["table"])
        if c:
            rec["frac_ceiling"] = round((q["gbs"] if bound == "hbm" else q["tops"]) / c, 4)
        rec["tile"] = "%dx%dx%d" % (q["info"]["block_m"], q["info"]["block_n"], q["info"]["block_k"])
        rec["mfma_block"] = q["info"]["mfma_block"]
        rec["occupancy"] = q["occupancy"]
        return rec

    record = {
        "workload": desc, "M": M, "N": N, "K": K, "dtype": dtype, "layout": layout, "bound": bound,
        "value": round(value, 2), "unit": vunit, "best": pair_key(*best), "ms_per_step": round(r["ms_per_step"], 5),
        "tile": "%dx%dx%d" % (info["block_m"], info["block_n"], info["block_k"]),
        "lds_bytes": info["lds_bytes"], "grid": info["grid"], "splits": info["splits"],
        "sk_tiles": info["sk_tiles"], "mfma_block": info["mfma_block"], "roofline": roof,
        "pairs_bit_identical": identical,
        "data": "synthetic (seeded), inputs resident in HBM, rotated over %d sets (%.0f MiB)" % (
            nrot, nrot * set_bytes / 2 ** 20),
        "pairs": {pair_key(*p): pair_record(q) for p, q in results.items()},
    }
    if hot is not None:
        record["hot"] = hot
    del sets, a, b, first_c
    torch.cuda.empty_cache()
    return record


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--rounds", type=int, default=3, help="rounds over all pairs; each pair reports its median")
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOADS),
                    help="one workload, or all: the five benchmark workloads (headline int8 4096^3)")
    ap.add_argument("--pairs", default="all", help="comma list like 3:direct,2:reg, or all")
    ap.add_argument("--tile", default="auto", help="tile class: auto, 256x256, 256x256w8, 128x128, 32x64")
    ap.add_argument("--splits", type=int, default=1,
                    help="K splits per C tile (gemm_run_splitk); 0 = the library's choice")
    ap.add_argument("--streamk", action="store_true", help="time gemm_run_streamk instead of gemm_run")
    ap.add_argument("--sk-grid", type=int, default=0,
                    help="stream-K workgroups (gemm_run_streamk's grid; 0 = one per CU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling-probe", action="store_true",
                    help="take the ceilings from profiles/ceilings.txt instead of measuring them")
    ap.add_argument("--cpu-seconds", type=float, default=None,
                    help="CPU oracle budget per workload (default: 10 s for the headline workload, 3 s for "
                         "each other one)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this GEMM is measured on a single MI355X "
              "(--gpus %d requested); multi-GPU runs are not part of this build." % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    names = FIVE if args.workload == "all" else [args.workload]

    # The ceiling probe runs first, as a child process, before this process
    # touches the GPU.
    table = None if args.no_ceiling_probe else probe_ceilings()
    if table is not None:
        ceilings = {"table": table, "source": "ceiling_probe, same run and box (MFMA loop fed from LDS with "
                                              "random data, in the GEMM's block shape / HBM streaming read)"}
    else:
        ceilings = {"table": committed_ceilings(), "source": "profiles/ceilings.txt (committed ceiling_probe output)"}

    import torch
    from software_pipelined_tiled_02_amd import binding

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.pairs == "all":
        pairs = [(s, v) for s in (1, 2, 3, 4) for v in ("reg", "direct")]
    else:
        pairs = [(int(p.split(":")[0]), p.split(":")[1]) for p in args.pairs.split(",")]

    g = binding.Gemm(0)
    g.set_tile(args.tile)
    res_table = kernel_resources()
    configs = {}
    for name in names:
        configs[name] = measure_workload(name, args, g, ceilings, res_table, pairs)
    g.close()
    if not args.no_cpu_baseline:
        for name in names:
            M, N, K, dtype, layout, dist, scale, bound, desc = WORKLOADS[name]
            budget = args.cpu_seconds if args.cpu_seconds is not None else (
                10.0 if name == HEADLINE or len(names) == 1 else 3.0)
            configs[name]["cpu_baseline"] = cpu_baseline(M, N, K, dtype, layout, dist, scale, budget)

    head = configs[HEADLINE if HEADLINE in configs else names[0]]
    M, N, K = head["M"], head["N"], head["K"]
    best_s, best_v = head["best"][1:].split("_")
    line = {
        "metric": "GEMM TFLOP/s (int8 TOP/s) and % of MFMA peak per stage count/variant, 1 GPU",
        "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"i8": "int8", "f16": "fp16", "bf16": "bf16", "f32": "fp32"}[head["dtype"]],
        "data": head["data"],
        "config": {"workload": head["workload"], "M": M, "N": N, "K": K, "layout": head["layout"],
                   "stages": int(best_s), "variant": best_v, "tile": head["tile"],
                   "lds_bytes": head["lds_bytes"], "grid": head["grid"], "splits": head["splits"],
                   "sk_tiles": head["sk_tiles"], "mfma_block": head["mfma_block"]},
        "roofline": head["roofline"],
        "pairs_bit_identical": all(c["pairs_bit_identical"] for c in configs.values()),
        "rounds": args.rounds,
        "sweep": head["pairs"],
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if "hot" in head:
        line["hot"] = head["hot"]
    line["ceilings"] = {"source": ceilings["source"],
                        **{k: v for k, v in ceilings["table"].items() if k.startswith(("mfma", "hbm"))}}
    line["configs"] = configs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
