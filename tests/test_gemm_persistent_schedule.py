"""Model check of the persistent NVFP4 256x256 GEMM's load/store schedule (CPU).

gemm_nvfp4_w1_kernel runs a workgroup's tiles one after another through a
4-slot LDS ring. Per wave and stage it issues NIW direct global->LDS loads;
a tile's 16-byte C writes (64 per lane) go out after the next tile's first
four stages; vector-memory operations retire in issue order and `vmcnt(N)`
waits until at most N of them are in flight. `schedule` restates the
kernel's event order for one wave (all waves run the same sequence, and a
barrier completes every wave's earlier LDS reads):
  - the first tile's loads of stages 0-3 into slots 0-3;
  - per tile: the wait for its stage 0 (63 after a store, else the count
    for the stages loaded behind it), barrier, reads of stage 0;
  - per stage `it`: the wait for the stream's next stage (63 in the first
    three stages after a store; two stages behind it when the stream runs
    on, one or none near the end), barrier, the refill of stage it's slot
    with stage it+4 or, with `ahead`, the next tile's stage it+4-nk, then
    the reads of the next stage;
  - at the tile's end: without `ahead`, a barrier and the next tile's
    stages 0-3 into the slots that follow; then the store (64 writes, or
    checked writes that are waited for at once).
The test checks, over tile sequences, K lengths and store forms, that:
  1. every wait leaves the stage it waits for retired (N is at most the
     number of operations issued after that stage's loads);
  2. every read finds, in its slot, the stage it expects, retired;
  3. no slot is refilled before a barrier that follows every read of the
     stage it held;
  4. every wait count fits the 6-bit vmcnt field.
"""
import itertools

import pytest

S = 4          # ring slots
NIW = 12       # loads per wave and stage
NST = 64       # 16-byte C writes per lane and tile


def schedule(nk, tiles):
    """Events of one wave. `tiles`: per tile (interior, fast_store); interior
    tiles may load ahead into the next tile when it is interior too."""
    ev = []
    nt = len(tiles)

    def ahead_of(t):
        return nk >= S and t + 1 < nt and tiles[t][0] and tiles[t + 1][0]

    slot = 0
    for s in range(min(S, nk)):
        ev.append(("dma", (0, s), s))
    stored = False
    for t in range(nt):
        ahead = ahead_of(t)
        if stored:
            n = 63
        elif nk >= 4:
            n = 3 * NIW
        elif nk == 3:
            n = 2 * NIW
        elif nk == 2:
            n = NIW
        else:
            n = 0
        ev.append(("wait", n, (t, 0)))
        ev.append(("barrier",))
        ev.append(("read", (t, 0), slot))
        for it in range(nk):
            more = it + 1 < nk
            nxt = (slot + 1) % S
            if more or ahead:
                if stored and it < S - 1:
                    n = 63
                elif ahead or it + 3 < nk:
                    n = 2 * NIW
                elif it + 2 < nk:
                    n = NIW
                else:
                    n = 0
                need = (t, it + 1) if more else (t + 1, 0)
                ev.append(("wait", n, need))
                ev.append(("barrier",))
            own = it + S < nk
            if own:
                ev.append(("dma", (t, it + S), slot))
            elif ahead:
                ev.append(("dma", (t + 1, it + S - nk), slot))
            if more:
                ev.append(("read", (t, it + 1), nxt))
            elif ahead:
                ev.append(("read", (t + 1, 0), nxt))
            slot = nxt
        if t + 1 < nt:
            if not ahead:
                ev.append(("wait", 63, None))
                ev.append(("barrier",))
                for s in range(min(S, nk)):
                    ev.append(("dma", (t + 1, s), (slot + s) % S))
        fast = tiles[t][1]
        if fast:
            ev.extend([("store",)] * NST)
        else:
            ev.append(("store",))
            ev.append(("wait", 0, None))
        stored = fast
    return ev


def check(ev):
    ops = []          # issued vector-memory operations, in order: ("dma", stage) or ("store",)
    retired = 0       # ops[:retired] have retired
    dma_at = {}       # stage -> index in ops
    content = {}      # slot -> stage its last load brought
    last_read = {}    # stage -> event index of its last read
    last_barrier = -1
    for i, e in enumerate(ev):
        kind = e[0]
        if kind == "dma":
            stage, slot = e[1], e[2]
            old = content.get(slot)
            if old is not None and old in last_read:
                assert last_barrier > last_read[old], f"slot {slot} refilled with {stage} before every read of {old}"
            content[slot] = stage
            dma_at[stage] = len(ops)
            for _ in range(NIW):
                ops.append(("dma", stage))
        elif kind == "store":
            ops.append(("store",))
        elif kind == "wait":
            n, need = e[1], e[2]
            assert 0 <= n <= 63, f"wait count {n}"
            retired = max(retired, len(ops) - n)
            if need is not None:
                last = dma_at[need] + NIW - 1
                assert last < retired, f"wait({n}) leaves stage {need} in flight"
        elif kind == "barrier":
            last_barrier = i
        elif kind == "read":
            stage, slot = e[1], e[2]
            assert content.get(slot) == stage, f"read of {stage} finds {content.get(slot)} in slot {slot}"
            assert dma_at[stage] + NIW - 1 < retired, f"read of {stage} before its loads retired"
            last_read[stage] = i


@pytest.mark.parametrize("nk", [1, 2, 3, 4, 5, 6, 7, 8, 9, 33, 65])
def test_schedule_invariants(nk):
    kinds = [(True, True), (True, False), (False, True), (False, False)]
    for nt in (1, 2, 3):
        for tiles in itertools.product(kinds, repeat=nt):
            check(schedule(nk, list(tiles)))


def test_long_interior_run():
    # a workgroup with many interior tiles: the stream runs on through all
    for nk in (4, 32, 65):
        check(schedule(nk, [(True, True)] * 7))


def test_model_catches_a_short_wait():
    # the model is not vacuous: wait(63) after a store that issued fewer
    # than 63 writes (the checked form, had it not been waited for) leaves
    # the stage it waits for in flight
    ev = schedule(8, [(True, True), (True, True)])
    first = next(k for k, e in enumerate(ev) if e[0] == "store")
    bad = ev[:first] + [("store",)] * 8 + ev[first + NST:]
    with pytest.raises(AssertionError, match="in flight"):
        check(bad)
    # and a refill moved before its barrier is flagged
    j = next(k for k, e in enumerate(ev) if e[0] == "dma" and e[1] == (0, 4))
    moved = list(ev)
    moved[j - 1], moved[j] = moved[j], moved[j - 1]
    with pytest.raises(AssertionError):
        check(moved)
