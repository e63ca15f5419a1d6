"""Model check of the MX-FP4 256x256 GEMMs' load schedules (CPU).

gemm_mxfp4_w1p_kernel (K % 512 == 0) runs a workgroup's tiles one after
another, each a stream of nk 128-element stages through a 4-slot LDS ring
of codes and a 3-slot ring of scale groups (group g of a tile holds the
scales of its stages 4g .. 4g+3). Per wave, stage it's refill (after the
barrier in its row 4) loads the codes of stage it+4 and its part of scale
group it/4 + 2: one 16-byte load in stages it % 4 == 0 (A rows) and 2 (B
rows). gemm_mxfp4_w1_kernel (other K) runs one tile per workgroup with
two 4-byte scale loads in every stage: the model's single-tile quad-lane
case. Past the tile's end these are the next tile's first stages and
groups when the stream runs on (`ahead`: whole groups, at least two, both
tiles interior), else the tile's last stage or group again (never read). A tile's prologue
(first tile, or after a tile that did not stream on: every load waited for
first) loads group 0, then stages 0-3 with their parts of group 1. A
tile's store (64 writes, or checked writes waited for at once) follows the
next tile's first loads. Loads and stores retire in issue order; vmcnt(N)
waits until at most N are in flight. `schedule` restates the kernel's event
order for one wave, slots worked out as the kernel does (every wave runs
the same sequence; a barrier completes every wave's earlier reads, and the
waves' equal waits make a group whole when this wave's part has landed).
The test checks that:
  1. every read finds its stage's codes and scale group in the slots it
     uses, landed (the group with both parts, or all eight);
  2. no slot of either ring is refilled before a barrier that follows every
     read of what it held;
  3. every load's source lies in its tile (stage < nk, group < nk / 4 for
     the 16-byte loads, which read a row's 16 bytes at 16 g);
  4. wait counts fit vmcnt.
"""
import itertools

import pytest

S, NG = 4, 3
CODES = 8      # code loads per wave and stage
NST = 64       # 16-byte C writes per lane and tile


def schedule(nk, tiles, wg, wait_loop=None, min_groups_ahead=2):
    """Events of one wave. `tiles`: per tile (interior, fast_store)."""
    ng = nk // 4
    niw2 = 2 * CODES + (1 if wg else 4)
    wait_loop = niw2 if wait_loop is None else wait_loop
    wait_first = niw2 + CODES + (0 if wg else 2)
    nt = len(tiles)
    ev = []

    def code(t, stage, slot):
        ev.append(("cdma", slot, (t, stage)))

    def scale(t, gi, part, gs):
        ev.append(("sdma", gs, (t, gi), part))

    def prologue(t):
        if wg:
            scale(t, 0, "A", 0)
            scale(t, 0, "B", 0)
        else:
            for p in range(4):
                for k in range(2):
                    scale(t, 0, (p, k), 0)
        for s in range(S):
            code(t, min(s, nk - 1), s)
            if wg:
                if s % 2 == 0:
                    scale(t, min(1, ng - 1), "A" if s % 4 == 0 else "B", 1)
            else:
                for k in range(2):
                    scale(t, 1, (s, k), 1)

    def ahead_of(t):
        return wg and ng >= min_groups_ahead and t + 1 < nt and tiles[t][0] and tiles[t + 1][0]

    prologue(0)
    slot, gb, stored, have0 = 0, 0, False, False
    for t in range(nt):
        ahead = ahead_of(t)
        if not have0:
            ev.append(("wait", 63 if stored else wait_first))
            ev.append(("barrier",))
            ev.append(("read", (t, 0), slot, gb))
        for it in range(nk):
            nxt = (slot + 1) % S
            gr = (gb + (it + 1) // 4) % NG
            ev.append(("wait", 63 if stored and it < S - 1 else wait_loop))
            ev.append(("barrier",))
            st = it + S
            own = st < nk
            code(t, st, slot) if own else code(t + 1, st - nk, slot) if ahead else code(t, nk - 1, slot)
            gi = it // 4 + 2
            gs = (gb + gi) % NG
            if wg:
                if it % 2 == 0:
                    part = "A" if it % 4 == 0 else "B"
                    if gi < ng:
                        scale(t, gi, part, gs)
                    elif ahead:
                        scale(t + 1, min(gi - ng, ng - 1), part, gs)
                    else:
                        scale(t, ng - 1, part, gs)
            else:
                for k in range(2):
                    scale(t, gi, (it % 4, k), gs)
            if it + 1 < nk:
                ev.append(("read", (t, it + 1), nxt, gr))
            elif ahead:
                ev.append(("read", (t + 1, 0), nxt, gr))
            slot = nxt
        last = t + 1 == nt
        if not last:
            if ahead:
                gb = (gb + ng) % NG
            else:
                ev.append(("wait", 0))
                ev.append(("barrier",))
                slot, gb = 0, 0
                prologue(t + 1)
            have0 = ahead
        else:
            ev.append(("wait", 0))
            ev.append(("barrier",))
        if tiles[t][1]:
            ev.extend([("store",)] * NST)
        else:
            ev.append(("store",))
            ev.append(("wait", 0))
        stored = tiles[t][1]
    return ev, nk, wg


def check(sched):
    ev, nk, wg = sched
    ng = nk // 4
    nparts = 2 if wg else 8
    ops, retired = [], 0
    code_slot, code_at = {}, {}
    gslot, gparts = {}, {}
    last_read, last_barrier = {}, -1
    for i, e in enumerate(ev):
        kind = e[0]
        if kind == "cdma":
            slot, src = e[1], e[2]
            assert 0 <= src[1] < nk, f"code load of stage {src} outside its tile"
            old = code_slot.get(slot)
            if old is not None and ("c", slot, old) in last_read:
                assert last_barrier > last_read[("c", slot, old)], f"code slot {slot} refilled before its reads"
            code_slot[slot] = src
            ops.extend([None] * CODES)
            code_at[(slot, src)] = len(ops) - 1
        elif kind == "sdma":
            gs, src, part = e[1], e[2], e[3]
            if wg:
                assert 0 <= src[1] < ng, f"16-byte scale load of group {src} outside its tile"
            old = gslot.get(gs)
            if old != src:
                if old is not None and ("g", gs, old) in last_read:
                    assert last_barrier > last_read[("g", gs, old)], f"group slot {gs} refilled before its reads"
                gslot[gs], gparts[gs] = src, {}
            ops.append(None)
            gparts[gs][part] = len(ops) - 1
        elif kind == "store":
            ops.append(None)
        elif kind == "wait":
            assert 0 <= e[1] <= 63, f"wait count {e[1]}"
            retired = max(retired, len(ops) - e[1])
        elif kind == "barrier":
            last_barrier = i
        elif kind == "read":
            stage, slot, gs = e[1], e[2], e[3]
            assert code_slot.get(slot) == stage, f"read of {stage} finds {code_slot.get(slot)} in code slot {slot}"
            assert code_at[(slot, stage)] < retired, f"codes of {stage} in flight"
            grp = (stage[0], stage[1] // 4)
            assert gslot.get(gs) == grp, f"read of {stage} finds group {gslot.get(gs)} in slot {gs}"
            assert len(gparts[gs]) == nparts, f"group {grp} incomplete"
            assert all(at < retired for at in gparts[gs].values()), f"group {grp} in flight"
            last_read[("c", slot, stage)] = i
            last_read[("g", gs, grp)] = i


KINDS = [(True, True), (True, False), (False, True), (False, False)]


@pytest.mark.parametrize("nk", [4, 8, 12, 20, 32])
def test_whole_groups(nk):
    for nt in (1, 2, 3):
        for tiles in itertools.product(KINDS, repeat=nt):
            check(schedule(nk, list(tiles), True))


@pytest.mark.parametrize("nk", [1, 2, 3, 4, 5, 7, 9, 20])
def test_quad_lane_groups(nk):
    # the one-tile kernel
    for tile in KINDS:
        check(schedule(nk, [tile], False))


def test_long_interior_run():
    for nk in (8, 12, 32, 64):
        check(schedule(nk, [(True, True)] * 6, True))


def test_model_catches_mistakes():
    # a loop wait one load looser than the kernel's
    with pytest.raises(AssertionError, match="in flight"):
        check(schedule(20, [(True, True)] * 2, True, wait_loop=18))
    # streaming on from a tile of one group: the next tile's group 0 is never loaded
    with pytest.raises(AssertionError, match="group"):
        check(schedule(4, [(True, True)] * 2, True, min_groups_ahead=1))
