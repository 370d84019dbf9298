"""Waits for the inline-assembly transposing reads, checked in this repo's own
gfx950 assembly (no GPU).

Layout RR's direct-to-LDS kernels read B fragments with ds_read_b64_tr_b16 /
_tr_b8 written as inline assembly (with LDS-DMA writes in flight the compiler
would otherwise drain every load before each of them).  The compiler does not
track their results, so the kernel waits for them explicitly.  This test
compiles the RR direct instances of tests/host/rr_asm_instances.hip to
assembly and replays each kernel's instruction stream: LDS (and scalar
memory) operations retire in issue order, `s_waitcnt lgkmcnt(N)` retires all
but the newest N, and no instruction other than another LDS access may read
or write a register a transposing read has not yet delivered.  The replay is
a dataflow over the kernel's control-flow graph (the outstanding-operation
queues of all paths into a block are joined, to a fixed point), so reads
issued at the end of a loop iteration are checked against the next one.  A
copy of the assembly with the explicit waits deleted must fail the same
check.
"""
import os
import re
import subprocess
import tempfile

import pytest

from tests.conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SRC = os.path.join(ROOT, "tests", "host", "rr_asm_instances.hip")
INC = [os.path.join(ROOT, "include"), os.path.join(ROOT, "software_pipelined_tiled_02_amd", "csrc")]

VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def vregs(text):
    out = set()
    for m in VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def functions(asm):
    """{kernel symbol: [(kind, text)]} with kind 'label' or 'inst'."""
    funcs, cur = {}, None
    for raw in asm.splitlines():
        line = raw.split(";")[0].rstrip()
        m = re.match(r"^(_ZN2pg15pipegemm_kernel\w+):", line)
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is None or not line.strip():
            continue
        s = line.strip()
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        if re.match(r"^\.?L?\w+:$", s):
            cur.append(("label", s[:-1]))
        elif not s.startswith("."):
            cur.append(("inst", s))
    return funcs


def blocks(insts):
    """Basic blocks of a kernel's instruction list: [(name, [instructions],
    [successor names])]."""
    out, cur, name, n = [], [], "entry", 0

    def close(succ):
        nonlocal cur, name, n
        out.append((name, cur, succ))
        n += 1
        cur, name = [], "_b%d" % n

    for kind, text in insts:
        if kind == "label":
            if cur or name != "entry" or out:
                close([text])
            name = text
            continue
        cur.append(text)
        mnem, _, ops = text.partition(" ")
        if mnem == "s_branch":
            close([ops.strip()])
        elif mnem.startswith("s_cbranch_"):
            close([ops.strip(), None])          # None: fall through
        elif mnem in ("s_endpgm", "s_setpc_b64"):
            close([])
    if cur:
        close([])
    # fall-through successors
    res = []
    for i, (nm, ins, succ) in enumerate(out):
        nxt = out[i + 1][0] if i + 1 < len(out) else None
        res.append((nm, ins, [nxt if x is None else x for x in succ if (x is not None or nxt is not None)]))
    return res


def transfer(fifo, ins, bad, where):
    """Replay one block from FIFO state `fifo` (a tuple of frozensets of
    pending transposing-read destinations, or empty sets for other LDS /
    scalar-memory operations, oldest first); collect violations."""
    fifo = list(fifo)
    for i, text in enumerate(ins):
        mnem, _, ops = text.partition(" ")
        if mnem == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", ops)
            if m:
                n = int(m.group(1))
                if len(fifo) > n:
                    fifo = fifo[len(fifo) - n:] if n else []
            continue
        pending = set().union(*fifo) if fifo else set()
        if mnem.startswith("ds_"):
            if mnem.startswith("ds_read_b64_tr"):
                dest, _, rest = ops.partition(",")
                if vregs(rest) & pending:
                    bad.add((where, i, text))
                fifo.append(frozenset(vregs(dest)))
            else:
                fifo.append(frozenset())
        elif mnem.startswith(("s_load", "s_buffer_load")):
            fifo.append(frozenset())
        elif vregs(ops) & pending:
            bad.add((where, i, text))
        fifo = fifo[-64:]
    return tuple(fifo)


def merge(a, b):
    """Join of two states: aligned at the newest entry, each position the
    union (lgkmcnt(N) retires all but the newest N)."""
    n = max(len(a), len(b))
    a = (frozenset(),) * (n - len(a)) + a
    b = (frozenset(),) * (n - len(b)) + b
    return tuple(x | y for x, y in zip(a, b))


def check(insts):
    """Violations: instructions that read or write a register an
    outstanding transposing read has not delivered, on any path."""
    bl = blocks(insts)
    index = {nm: k for k, (nm, _, _) in enumerate(bl)}
    state_in = {0: ()}
    work = [0]
    bad = set()
    while work:
        k = work.pop()
        nm, ins, succ = bl[k]
        out = transfer(state_in[k], ins, bad, nm)
        for s in succ:
            j = index.get(s)
            if j is None:
                continue
            new = merge(state_in[j], out) if j in state_in else out
            if state_in.get(j) != new:
                state_in[j] = new
                work.append(j)
    return sorted(bad)


@pytest.fixture(scope="module")
def asm():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "rr.s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "--cuda-device-only", "-S", SRC, "-o", out] + ["-I" + p for p in INC]
        subprocess.run(cmd, check=True, capture_output=True)
        return open(out).read()


def test_every_transposing_read_is_waited_for(asm):
    funcs = functions(asm)
    assert len(funcs) == 5, sorted(funcs)
    for name, insts in funcs.items():
        n_tr = sum(1 for k, t in insts if k == "inst" and t.startswith("ds_read_b64_tr"))
        assert n_tr > 0, name
        bad = check(insts)
        assert not bad, "%s: %s" % (name, bad[:3])


def test_deleted_waits_are_caught(asm):
    """Planted mistake: the kernel's explicit LDS waits removed from the
    assembly of the 16x16-block instances must be reported."""
    funcs = functions(asm)
    hit = 0
    for name in ("_ZN2pg15pipegemm_kernelILi1ELi0ELi0ELi3ELi1EEEvNS_8GemmArgsE",
                 "_ZN2pg15pipegemm_kernelILi0ELi0ELi0ELi2ELi1EEEvNS_8GemmArgsE",
                 "_ZN2pg15pipegemm_kernelILi2ELi0ELi0ELi4ELi1EEEvNS_8GemmArgsE"):
        insts = [(k, t) for k, t in funcs[name] if not (k == "inst" and re.match(r"s_waitcnt .*lgkmcnt", t))]
        hit += bool(check(insts))
    assert hit == 3
