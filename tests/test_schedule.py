"""Pipeline schedule simulator (no GPU): a logical race detector for the
K-loop schedules in csrc/gemm_kernel.h.

Each schedule is written out here as the sequence of events one wave
executes -- global loads into an LDS slot or a register set (in two halves,
as the kernel issues them), `s_waitcnt vmcnt(n)`, LDS stores from a register
set, barriers, and fragment reads of a slot -- mirroring the kernel's loops
event for event.  All waves run the same sequence, so the analysis works in
barrier epochs: an LDS-DMA write may land at any time between its issue and
the wait that covers it, and a read in epoch e is safe only if the slot's
last write is the expected tile, landed in an earlier epoch, and no write to
that slot is in flight or issued during epoch e by any wave.  Register sets
must never be reloaded before their tile has been stored to LDS.

The checks run for every variant, stage count 1-4 and tile count 1-12, and
the planted mistakes the skill lists (off-by-one slot, missing drain, wrong
wait, missing barrier) must each be caught.  This verifies the schedule;
the GPU marker-tile tests verify the compiled kernel.
"""
import pytest

LPT = 4          # loads per tile (any even number: the kernel issues two halves)
HALF = LPT // 2


class Violation(AssertionError):
    pass


def direct_program(S, nt, fault=None):
    ev = []
    if S == 1:
        ev.append(("load", 0, 0, 0, LPT))
        for kt in range(nt):
            ev.append(("wait", 0 if fault != "wait" else LPT))
            ev.append(("barrier",))
            ev.append(("read", 0, kt))
            if fault != "barrier":
                ev.append(("barrier",))
            ev.append(("load", kt + 1, 0, 0, LPT))
        if fault != "drain":
            ev.append(("wait", 0))
        return ev
    for t in range(S - 1):
        ev.append(("load", t, t, 0, LPT))
    ev.append(("wait", (S - 2) * LPT + (LPT if fault == "wait" else 0)))
    ev.append(("barrier",))
    ev.append(("read", 0, 0))
    ev.append(("load", S - 1, S - 1, 0, HALF))
    slot = 0
    for kt in range(nt):
        prev = (slot - 1) % S
        nxt = (slot + 1) % S
        if fault == "slot":
            prev = slot          # refill the slot being multiplied
        ev.append(("read", slot, kt))                      # steps 1..KSTEPS-1
        ev.append(("load", kt + S - 1, prev, HALF, LPT))   # second half
        ev.append(("wait", (S - 2) * LPT + (LPT if fault == "wait" else 0)))
        if fault != "barrier":
            ev.append(("barrier",))
        ev.append(("read", nxt, kt + 1))                   # next tile's step 0
        ev.append(("load", kt + S, slot, 0, HALF))         # first half
        slot = nxt
    if fault != "drain":
        ev.append(("wait", 0))
    return ev


def split_program(nt, fault=None):
    """The 3-stage direct ring of the 256x256 tiles, split by operand: A
    slots ("A", t % 3), B slots ("B", t % 2).  Loads carry LA = LB = HALF
    chunks each.  While tile kt is multiplied the A tile of kt+2 is loaded;
    after the barrier that ends tile kt, the B tile of kt+2."""
    ev = []
    for t in range(2):                                      # prologue: tiles 0 and 1
        ev.append(("load", t, ("A", t % 3), 0, HALF))
        ev.append(("load", t, ("B", t % 2), HALF, LPT))
    ev.append(("wait", LPT))
    ev.append(("barrier",))
    ev.append(("read", ("A", 0), 0))
    ev.append(("read", ("B", 0), 0))
    for kt in range(nt):
        ev.append(("read", ("A", kt % 3), kt))              # steps 1..KSTEPS-1
        ev.append(("read", ("B", kt % 2), kt))
        a_slot = (kt + 1) % 3 if fault == "slot" else (kt + 2) % 3
        ev.append(("load", kt + 2, ("A", a_slot), 0, HALF))
        ev.append(("wait", LPT if fault == "wait" else HALF))
        if fault != "barrier":
            ev.append(("barrier",))
        ev.append(("read", ("A", (kt + 1) % 3), kt + 1))    # next tile's step 0
        ev.append(("read", ("B", (kt + 1) % 2), kt + 1))
        b_slot = (kt + 1) % 2 if fault == "bslot" else kt % 2
        ev.append(("load", kt + 2, ("B", b_slot), HALF, LPT))
    if fault != "drain":
        ev.append(("wait", 0))
    return ev


def reg_program(S, nt, fault=None):
    ev = []
    if S == 1:
        ev.append(("gload", 0, 0, 0, LPT))
        ev.append(("swrite", 0, 0))
        ev.append(("barrier",))
        ev.append(("read", 0, 0))
        ev.append(("gload", 1, 0, 0, HALF))
        for kt in range(nt):
            ev.append(("read", 0, kt))
            ev.append(("gload", kt + 1, 0, HALF, LPT))
            if fault != "barrier":
                ev.append(("barrier",))
            ev.append(("swrite", 0, 0))
            ev.append(("barrier",))
            ev.append(("read", 0, kt + 1))
            ev.append(("gload", kt + 2, 0, 0, HALF))
        return ev
    R = S - 1
    for t in range(R):
        ev.append(("gload", t, t, 0, LPT))
    ev.append(("swrite", 0, 0))
    ev.append(("barrier",))
    ev.append(("read", 0, 0))
    ev.append(("gload", R, 0, 0, HALF))
    ntp = -(-nt // R) * R            # whole groups of R tiles
    for kt in range(ntp):
        i = kt % R
        nxt_set = (i + 1) % R
        if fault == "slot":
            nxt_set = i
        ev.append(("read", kt & 1, kt))
        ev.append(("gload", kt + R, i, HALF, LPT))
        ev.append(("swrite", nxt_set, (kt + 1) & 1))
        if fault != "barrier":
            ev.append(("barrier",))
        ev.append(("read", (kt + 1) & 1, kt + 1))
        ev.append(("gload", kt + 1 + R, nxt_set, 0, HALF))
    return ev


def check(events, nt, S):
    """Raise Violation if any read could see a stale or racing slot."""
    epoch = 0
    loads = []                      # [tile, slot, n_loads, issue_epoch, landed_epoch or None]
    slot_writes = {}                # slot -> list of (tile, issue_epoch, load record or None)
    sets = {}                       # set -> {"tile": t, "parts": set(), "stored": bool}
    reads = []
    for ev in events:
        kind = ev[0]
        if kind == "barrier":
            epoch += 1
        elif kind == "load":
            _, tile, slot, j0, j1 = ev
            rec = [tile, slot, j1 - j0, epoch, None]
            loads.append(rec)
            slot_writes.setdefault(slot, []).append((tile, epoch, rec))
        elif kind == "wait":
            allowed = ev[1]
            pending = 0
            for rec in reversed(loads):
                if rec[4] is None:
                    pending += rec[2]
                    if pending > allowed:
                        rec[4] = epoch
            # every load older than the allowed window has landed
            out = 0
            for rec in reversed(loads):
                out += rec[2]
                if out > allowed and rec[4] is None:
                    rec[4] = epoch
        elif kind == "gload":
            _, tile, st, j0, j1 = ev
            cur = sets.get(st)
            if cur is not None and cur["tile"] != tile and not cur["stored"] and cur["tile"] < nt:
                raise Violation("register set %d reloaded before tile %d was stored" % (st, cur["tile"]))
            if cur is None or cur["tile"] != tile:
                cur = {"tile": tile, "parts": set(), "stored": False}
                sets[st] = cur
            cur["parts"].update(range(j0, j1))
        elif kind == "swrite":
            _, st, slot = ev
            cur = sets.get(st)
            if cur is None or len(cur["parts"]) != LPT:
                raise Violation("LDS store from an incomplete register set %d" % st)
            cur["stored"] = True
            slot_writes.setdefault(slot, []).append((cur["tile"], epoch, None))
        elif kind == "read":
            reads.append((ev[1], ev[2], epoch))
    seen = set()
    for slot, tile, e in reads:
        if tile >= nt:
            continue                # the hand-over after the last tile reads unused data
        seen.add(tile)
        writes = slot_writes.get(slot, [])
        done = [w for w in writes if w[1] < e and (w[2] is None or (w[2][4] is not None and w[2][4] < e))]
        racing = [w for w in writes if w[1] <= e and w not in done]
        if racing:
            raise Violation("read of slot %s (tile %d) in epoch %d races with a write of tile %d"
                            % (slot, tile, e, racing[0][0]))
        # the last landed write must be this tile (both halves for LDS-DMA)
        last = [w for w in done if w[0] == done[-1][0]] if done else []
        if not done or done[-1][0] != tile:
            raise Violation("read of slot %s in epoch %d sees tile %s, wants %d"
                            % (slot, e, done[-1][0] if done else None, tile))
        need = HALF if isinstance(slot, tuple) else LPT      # one operand's chunks, or both
        if last and last[0][2] is not None and sum(w[2][2] for w in last) != need:
            raise Violation("tile %d only partly in slot %s" % (tile, slot))
    if seen != set(range(nt)):
        raise Violation("tiles never multiplied: %s" % sorted(set(range(nt)) - seen))
    # no LDS-DMA load -- including the all-zero ones past the last tile --
    # may still be writing LDS when the loop ends
    if any(rec[4] is None for rec in loads):
        raise Violation("an LDS-DMA load was never waited for")
    return True


@pytest.mark.parametrize("variant", ["direct", "reg"])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
def test_schedules_are_race_free(variant, S):
    for nt in range(1, 13):
        prog = direct_program(S, nt) if variant == "direct" else reg_program(S, nt)
        check(prog, nt, S)


@pytest.mark.parametrize("variant,S,fault", [
    ("direct", 2, "slot"), ("direct", 3, "slot"), ("direct", 4, "slot"),
    ("direct", 1, "wait"), ("direct", 2, "wait"), ("direct", 4, "wait"),
    ("direct", 1, "barrier"), ("direct", 3, "barrier"),
    ("reg", 1, "barrier"), ("reg", 2, "barrier"), ("reg", 3, "slot"), ("reg", 4, "slot"),
])
def test_planted_schedule_mistakes_are_caught(variant, S, fault):
    caught = False
    for nt in range(1, 13):
        prog = direct_program(S, nt, fault) if variant == "direct" else reg_program(S, nt, fault)
        try:
            check(prog, nt, S)
        except Violation:
            caught = True
            break
    assert caught, (variant, S, fault)


def test_missing_drain_wait_is_caught():
    with pytest.raises(Violation):
        check(direct_program(3, 1, "drain"), 1, 3)


def test_split_ring_is_race_free():
    for nt in range(1, 13):
        check(split_program(nt), nt, 3)


@pytest.mark.parametrize("fault", ["slot", "bslot", "wait", "barrier", "drain"])
def test_split_ring_mistakes_are_caught(fault):
    caught = False
    for nt in range(1, 13):
        try:
            check(split_program(nt, fault), nt, 3)
        except Violation:
            caught = True
            break
    assert caught, fault
