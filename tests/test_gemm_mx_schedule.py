"""Model check of the MX-FP4 256x256 GEMM's load schedule (CPU).

gemm_mxfp4_w1_kernel streams a K range of nk 128-element stages through a
4-slot LDS ring of codes and a 3-slot ring of scale groups (group g holds
the scales of stages 4g .. 4g+3). Per wave, stage it's refill (after the
barrier in its row 4) loads the codes of stage it+4 (the last stage again
past the end) and its part of scale group it/4 + 2: with whole groups (WG)
one 16-byte load in stages it % 4 == 0 (A rows) and 2 (B rows), otherwise
two 4-byte loads in every stage. The prologue loads group 0, then stages
0-3 with their parts of group 1. Loads retire in issue order; vmcnt(N) waits
until at most N are in flight. `schedule` restates the kernel's event order
for one wave (every wave runs the same sequence; a barrier completes every
wave's earlier reads, and the waves' equal waits make a group whole when
this wave's part of it has landed). The test checks that every read finds
its stage's codes and its group in the slots, landed, that no slot of
either ring is refilled before a barrier that follows every read of what
it held, and that wait counts fit vmcnt.
"""
import pytest

S, NG = 4, 3
CODES = 8      # code loads per wave and stage


def parts(wg, it):
    """Scale loads of stage it's refill: (group offset, part) pairs."""
    if wg:
        return [("A",)] if it % 4 == 0 else [("B",)] if it % 4 == 2 else []
    return [(it % 4, 0), (it % 4, 1)]


def schedule(nk, wg, wait_loop=None, wait_first=None):
    niw = CODES + (1 if wg else 2)
    niw2 = 2 * CODES + (1 if wg else 4)
    wait_loop = niw2 if wait_loop is None else wait_loop
    wait_first = niw2 + CODES + (0 if wg else 2) if wait_first is None else wait_first
    last_group = (nk - 1) // 4
    ev = []

    def scale(gi, part):
        # groups past the last reload it (WG) or repeat the last stage's words
        src = min(gi, last_group)
        ev.append(("sdma", gi % NG, (src, part), gi))

    def codes(stage, slot):
        ev.append(("cdma", slot, min(stage, nk - 1)))

    for p in parts(wg, 0) + parts(wg, 2) if wg else [(ph, t) for ph in range(4) for t in range(2)]:
        scale(0, p)
    for s in range(S):
        codes(s, s)
        for p in parts(wg, s):
            scale(1, p)
    ev.append(("wait", wait_first))
    ev.append(("barrier",))
    ev.append(("read", 0, 0))
    slot = 0
    for it in range(nk):
        ev.append(("wait", wait_loop))
        ev.append(("barrier",))
        codes(it + S, slot)
        for p in parts(wg, it):
            scale(it // 4 + 2, p)
        if it + 1 < nk:
            ev.append(("read", it + 1, (slot + 1) % S))
        slot = (slot + 1) % S
    return ev, wg


def check(sched):
    ev, wg = sched
    nparts = 2 if wg else 8
    ops, retired = [], 0
    code_at, code_slot = {}, {}
    gslot, gparts, gdone = {}, {}, {}
    last_read, last_barrier = {}, -1
    for i, e in enumerate(ev):
        if e[0] == "cdma":
            slot, stage = e[1], e[2]
            old = code_slot.get(slot)
            if old is not None and ("c", slot, old) in last_read:
                assert last_barrier > last_read[("c", slot, old)], f"code slot {slot} refilled before its reads"
            code_slot[slot] = stage
            ops.extend([None] * CODES)
            code_at[(slot, stage)] = len(ops) - 1
        elif e[0] == "sdma":
            gs, (src, part), gi = e[1], e[2], e[3]
            if gslot.get(gs) != gi:
                old = gslot.get(gs)
                if old is not None and ("g", gs, old) in last_read:
                    assert last_barrier > last_read[("g", gs, old)], f"group slot {gs} refilled before its reads"
                gslot[gs], gparts[gs] = gi, {}
            ops.append(None)
            gparts[gs][part] = (src, len(ops) - 1)
        elif e[0] == "wait":
            assert 0 <= e[1] <= 63
            retired = max(retired, len(ops) - e[1])
        elif e[0] == "barrier":
            last_barrier = i
        elif e[0] == "read":
            stage, slot = e[1], e[2]
            assert code_slot.get(slot) == stage, f"read of stage {stage} finds {code_slot.get(slot)}"
            assert code_at[(slot, stage)] < retired, f"codes of stage {stage} in flight"
            gi, gs = stage // 4, (stage // 4) % NG
            assert gslot.get(gs) == gi, f"read of stage {stage} finds group {gslot.get(gs)}"
            got = gparts[gs]
            assert len(got) == nparts, f"group {gi} incomplete"
            for part, (src, at) in got.items():
                assert src == gi, f"group {gi} part {part} holds group {src}"
                assert at < retired, f"group {gi} part {part} in flight"
            last_read[("c", slot, stage)] = i
            last_read[("g", gs, gi)] = i


@pytest.mark.parametrize("nk", [4, 8, 12, 20, 64])
def test_whole_groups(nk):
    check(schedule(nk, True))


@pytest.mark.parametrize("nk", [1, 2, 3, 4, 5, 7, 9, 20])
def test_quad_lane_groups(nk):
    check(schedule(nk, False))


def test_model_catches_loose_waits():
    # Waits that allow more loads in flight than the trailing loads of later
    # stages leave the needed codes in flight. (The kernel's first wait, 25
    # with whole groups, also covers group 1's first part, which stage 0's
    # refill issues after its codes: 26 would still be safe; likewise the
    # scale loads that end a quad-lane refill.)
    check(schedule(20, True, wait_first=26))
    with pytest.raises(AssertionError, match="in flight"):
        check(schedule(20, True, wait_loop=18))
    with pytest.raises(AssertionError, match="in flight"):
        check(schedule(20, True, wait_first=27))
    check(schedule(20, False, wait_loop=22))
    with pytest.raises(AssertionError, match="in flight"):
        check(schedule(20, False, wait_loop=23))
