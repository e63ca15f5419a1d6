"""Model check of the persistent NVFP4 256x256 GEMM's load/store schedule (CPU).

gemm_nvfp4_w1_kernel runs a workgroup's tiles one after another through a
4-slot LDS ring of stage codes and a 3-slot ring of scale groups (a group
holds the scales of an even stage and the odd stage after it). Per wave, a
stage's refill issues NO direct global->LDS loads of codes, an even stage's
also the IS loads of its group (NE in all); a tile's 16-byte C writes (64
per lane) go out after the next tile's first four stages; vector-memory
operations retire in issue order and `vmcnt(N)` waits until at most N of
them are in flight. `schedule` restates the kernel's event order for one
wave (all waves run the same sequence, and a barrier completes every wave's
earlier LDS reads), with the ring slots worked out as the kernel does:
  - the first tile's loads of stages 0-3 into slots 0-3, groups 0, 0, 1, 1;
  - per tile: the wait for its stage 0 (63 after a store, else the count
    for the stages loaded behind it), barrier, reads of stage 0;
  - per stage `it`: the wait for the stream's next stage (63 in the first
    three stages after a store; two stages behind it when the stream runs
    on, one or none near the end), barrier, the refill of stage it's slot
    with stage it+4 or, with `ahead`, the next tile's stage it+4-nk (an
    even one into the group slot before stage it's), then the reads of the
    next stage;
  - at the tile's end: without `ahead`, a barrier and the next tile's
    stages 0-3 into the slots that follow; then the store (64 writes, or
    checked writes that are waited for at once).
The test checks, over tile sequences, K lengths and store forms, that:
  1. every wait leaves the stage it waits for retired, codes and scales
     (N is at most the number of operations issued after them);
  2. every read finds, in its slots, the stage and the scale group it
     expects, retired;
  3. no slot of either ring is refilled before a barrier that follows every
     read of what it held;
  4. every wait count fits the 6-bit vmcnt field.
"""
import itertools

import pytest

S = 4          # code ring slots
NG = 3         # scale group ring slots
NO = 8         # code loads per wave and stage
IS = 2         # scale loads per wave and group
NE = NO + IS   # loads of an even stage
NST = 64       # 16-byte C writes per lane and tile


def count(stage):
    return NE if stage[1] % 2 == 0 else NO


def schedule(nk, tiles, group_of_refill=lambda gq: (gq - 1) % NG):
    """Events of one wave. `tiles`: per tile (interior, fast_store); interior
    tiles may load ahead into the next tile when it is interior too. The
    kernel runs whole pairs of stages (nk even)."""
    assert nk % 2 == 0
    ev = []
    nt = len(tiles)

    def ahead_of(t):
        return nk >= S and t + 1 < nt and tiles[t][0] and tiles[t + 1][0]

    slot, gq = 0, 0
    for s in range(min(S, nk)):
        ev.append(("dma", (0, s), s, s >> 1))
    stored = False
    for t in range(nt):
        ahead = ahead_of(t)
        n = 63 if stored else NO + NE + NO if nk >= 4 else NO
        ev.append(("wait", n, (t, 0)))
        ev.append(("barrier",))
        ev.append(("read", (t, 0), slot, gq))
        for it in range(nk):
            more = it + 1 < nk
            nxt = (slot + 1) % S
            odd = it % 2 == 1
            gn = (gq + 1) % NG if odd else gq
            rgs = group_of_refill(gq)
            if more or ahead:
                if stored and it < S - 1:
                    n = 63
                elif ahead or it + 3 < nk:
                    n = NE + NO
                elif it + 2 < nk:
                    n = NO
                else:
                    n = 0
                need = (t, it + 1) if more else (t + 1, 0)
                ev.append(("wait", n, need))
                ev.append(("barrier",))
            own = it + S < nk
            if own:
                ev.append(("dma", (t, it + S), slot, rgs))
            elif ahead:
                ev.append(("dma", (t + 1, it + S - nk), slot, rgs))
            if more:
                ev.append(("read", (t, it + 1), nxt, gn))
            elif ahead:
                ev.append(("read", (t + 1, 0), nxt, gn))
            slot, gq = nxt, gn
        if t + 1 < nt:
            if not ahead:
                ev.append(("wait", 63, None))
                ev.append(("barrier",))
                for s in range(min(S, nk)):
                    ev.append(("dma", (t + 1, s), (slot + s) % S, gq if s < 2 else (gq + 1) % NG))
        fast = tiles[t][1]
        if fast:
            ev.extend([("store",)] * NST)
        else:
            ev.append(("store",))
            ev.append(("wait", 0, None))
        stored = fast
    return ev


def check(ev):
    ops = []          # issued vector-memory operations, in order
    retired = 0       # ops[:retired] have retired
    done_at = {}      # stage -> index in ops of its last load (codes, and the group's with an even stage)
    content = {}      # code slot -> stage its last load brought
    gcontent = {}     # group slot -> (tile, pair) its last load brought
    last_read = {}    # stage or ("pair", tile, pair) -> event index of its last read
    last_barrier = -1

    def landed(stage):
        pair_head = (stage[0], stage[1] - stage[1] % 2)   # the even stage whose loads bring the group
        return done_at[stage] < retired and done_at[pair_head] < retired

    for i, e in enumerate(ev):
        kind = e[0]
        if kind == "dma":
            stage, slot, gsl = e[1], e[2], e[3]
            old = content.get(slot)
            if old is not None and old in last_read:
                assert last_barrier > last_read[old], f"slot {slot} refilled with {stage} before every read of {old}"
            content[slot] = stage
            if stage[1] % 2 == 0:
                pair = (stage[0], stage[1] // 2)
                oldp = gcontent.get(gsl)
                if oldp is not None and ("pair",) + oldp in last_read:
                    assert last_barrier > last_read[("pair",) + oldp], \
                        f"group slot {gsl} refilled with {pair} before every read of {oldp}"
                gcontent[gsl] = pair
            ops.extend([("dma", stage)] * count(stage))
            done_at[stage] = len(ops) - 1
        elif kind == "store":
            ops.append(("store",))
        elif kind == "wait":
            n, need = e[1], e[2]
            assert 0 <= n <= 63, f"wait count {n}"
            retired = max(retired, len(ops) - n)
            if need is not None:
                assert landed(need), f"wait({n}) leaves stage {need} in flight"
        elif kind == "barrier":
            last_barrier = i
        elif kind == "read":
            stage, slot, gsl = e[1], e[2], e[3]
            pair = (stage[0], stage[1] // 2)
            assert content.get(slot) == stage, f"read of {stage} finds {content.get(slot)} in slot {slot}"
            assert gcontent.get(gsl) == pair, f"read of {stage} finds group {gcontent.get(gsl)} in slot {gsl}"
            assert landed(stage), f"read of {stage} before its loads retired"
            last_read[stage] = i
            last_read[("pair",) + pair] = i


@pytest.mark.parametrize("nk", [2, 4, 6, 8, 10, 34, 66])
def test_schedule_invariants(nk):
    kinds = [(True, True), (True, False), (False, True), (False, False)]
    for nt in (1, 2, 3):
        for tiles in itertools.product(kinds, repeat=nt):
            check(schedule(nk, list(tiles)))


def test_long_interior_run():
    # a workgroup with many interior tiles: the stream runs on through all
    for nk in (4, 32, 66):
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


def test_model_catches_a_wrong_group_slot():
    # refilling the group slot of the pair being read (instead of the one
    # before it) overwrites scales a later read still needs
    with pytest.raises(AssertionError, match="group"):
        check(schedule(8, [(True, True), (True, True)], group_of_refill=lambda gq: gq))
    with pytest.raises(AssertionError, match="group"):
        check(schedule(8, [(True, True)], group_of_refill=lambda gq: (gq + 1) % NG))


def test_model_catches_an_odd_stage_count_in_flight():
    # a wait that allowed two even stages' loads (NE + NE) behind the stage
    # it needs would leave part of that stage in flight
    ev = schedule(8, [(True, False)])
    k = next(k for k, e in enumerate(ev) if e[0] == "wait" and e[1] == NE + NO)
    bad = list(ev)
    bad[k] = ("wait", NE + NE, ev[k][2])
    with pytest.raises(AssertionError, match="in flight"):
        check(bad)
