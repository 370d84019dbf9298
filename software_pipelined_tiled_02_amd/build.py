"""Build libpipegemm.so (gfx950) in-tree with hipcc.

Each translation unit under csrc/ is compiled on its own (in parallel) and
the objects are linked into software_pipelined_tiled_02_amd/libpipegemm.so.
Each kernel's register, LDS and occupancy figures, as the compiler reports
them (its kernel-resource-usage remarks), are written to
kernel_resources.json beside the library.  Two standalone measurement
programs are built beside it: `ceiling_probe`
(csrc/ceiling_probe.hip: MFMA and HBM rates of the chip, no GEMM code) and
`lds_layout_probe` (csrc/lds_layout_probe.hip: LDS bank conflicts of the
fragment reads under three tile layouts).
"""
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpipegemm.so")
RESOURCES = os.path.join(HERE, "kernel_resources.json")
PROBES = ["ceiling_probe", "lds_layout_probe"]
SOURCES = ["abi.hip", "kernels_i8.hip", "kernels_f16.hip", "kernels_bf16.hip", "kernels_f32.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def build(jobs=None, verbose=False):
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    objs, procs, logs = [], [], {}
    pending = list(SOURCES)
    while pending or procs:
        while pending and len(procs) < jobs:
            src = pending.pop(0)
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        src, p = procs.pop(0)
        out, _ = p.communicate()
        logs[src] = out.decode(errors="replace")
        if p.returncode != 0:
            for _, q in procs:
                q.kill()
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, logs[src]))
    write_resources(logs)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for name in PROBES:
        exe = os.path.join(HERE, name)
        tmp = exe + ".tmp%d" % os.getpid()
        subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, name + ".hip"), "-o", tmp], check=True)
        os.replace(tmp, exe)
    return LIB


_KEYS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
         "Occupancy [waves/SIMD]": "waves_per_simd", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
         "LDS Size [bytes/block]": "lds_bytes"}


def parse_resource_remarks(text):
    """{kernel symbol: {figure: value}} from the compiler's
    kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*?): (\S+) \[-Rpass-analysis", line)
        if m and cur is not None and m.group(1) in _KEYS:
            v = m.group(2)
            cur[_KEYS[m.group(1)]] = int(v) if v.lstrip("-").isdigit() else v
    return out


def write_resources(logs):
    table = {}
    for text in logs.values():
        table.update({k: v for k, v in parse_resource_remarks(text).items() if "pipegemm_kernel" in k})
    tmp = RESOURCES + ".tmp%d" % os.getpid()
    with open(tmp, "w") as f:
        json.dump(table, f, indent=0, sort_keys=True)
    os.replace(tmp, RESOURCES)


def kernel_symbol(dtype, layout, tile, stages, variant):
    """Symbol of the kernel instance pg::pipegemm_kernel<dtype, layout, tile,
    stages, variant> (all enum values as integers)."""
    return "_ZN2pg15pipegemm_kernelILi%dELi%dELi%dELi%dELi%dEEEvNS_8GemmArgsE" % (dtype, layout, tile, stages, variant)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
