"""Model check of the LDS-DMA GEMM's stage ring (CPU).

The GEMM kernel stages its operands through an S-slot ring in LDS: stage k
lives in slot k % S; its loads (NIW direct global->LDS loads per wave) are
issued S-1 stages ahead; at the top of iteration `it` each wave waits until
at most N of its own loads are in flight (vmcnt counts them and they retire
in order) and the workgroup barriers; then the wave reads stage it's
fragments and refills the slot stage it-1 used with stage it+S-1, in either
order (the refill-after-read order is the FP8 one).

`schedule` restates that loop's event order for one wave (every wave runs
the same sequence); the test checks, for every ring depth, K length, loads
per stage and both refill orders, the invariants the kernel relies on:
  1. when a wave passes its wait at iteration it, none of its loads of
     stages <= it is still in flight (so after the barrier every wave's
     loads of stage it are in LDS);
  2. a refill of slot j % S with stage j is issued only after the barrier of
     an iteration > j - S, i.e. after every wave has finished reading the
     slot's previous stage j - S (each wave completes its LDS reads before
     it reaches a barrier: the wait also drains lgkmcnt);
  3. within an iteration, the slot being read is not the slot being
     refilled;
  4. every stage is loaded once and read once, from slot k % S, in order;
  5. the wait counts fit the 6-bit vmcnt field.
"""
import itertools

import pytest


def wait_count(S, nk, niw, it):
    # the kernel's choice of N for iteration it (stages issued after it:
    # ahead = min(S - 2, nk - 1 - it))
    ahead = min(S - 2, nk - 1 - it)
    if S > 2 and ahead >= S - 2:
        return niw * (S - 2)
    if S > 3 and ahead == 1:
        return niw
    return 0


def schedule(S, nk, niw, late):
    ev = []
    for s in range(S - 1):
        if s < nk:
            ev += [("issue", s, s % S)] * niw
    for it in range(nk):
        ev.append(("wait", wait_count(S, nk, niw, it), it))
        ev.append(("barrier", it))
        refill = [("issue", it + S - 1, (it + S - 1) % S)] * niw if it + S - 1 < nk else []
        read = [("read", it, it % S)]
        ev += (read + refill) if late else (refill + read)
    return ev


def check(S, nk, niw, late):
    ev = schedule(S, nk, niw, late)
    issued = []                              # stages of this wave's loads, in issue order
    it_now = -1
    read_slot_now = None
    refill_slots_now = []
    for e in ev:
        kind = e[0]
        if kind == "issue":
            _, stage, slot = e
            assert slot == stage % S
            if it_now >= 0:
                # 2: the slot's previous stage was read before this barrier
                assert stage - S <= it_now - 1, (S, nk, niw, late, e, it_now)
            else:
                assert stage < S - 1                     # prologue: fresh slots
            refill_slots_now.append(slot)
            issued.append(stage)
        elif kind == "wait":
            _, n, it = e
            assert 0 <= n <= 63                          # 5
            # 1: the loads possibly in flight are the last n issued; none is
            # of a stage <= it
            in_flight = issued[len(issued) - n:] if n else []
            assert all(s > it for s in in_flight), (S, nk, niw, late, it, in_flight)
            assert it in issued                         # stage it was issued at all
        elif kind == "barrier":
            # 3: checked at the end of the previous iteration
            if read_slot_now is not None:
                assert read_slot_now not in refill_slots_now
            it_now = e[1]
            read_slot_now, refill_slots_now = None, []
        elif kind == "read":
            _, stage, slot = e
            assert stage == it_now and slot == stage % S  # 4
            read_slot_now = slot
    if read_slot_now is not None:
        assert read_slot_now not in refill_slots_now
    # 4: each stage loaded by niw loads, once, in order
    assert issued == [s for s in range(nk) for _ in range(niw)]
    assert [e[1] for e in ev if e[0] == "read"] == list(range(nk))


@pytest.mark.parametrize("late", [False, True])
@pytest.mark.parametrize("S", [2, 3, 4, 5])
def test_ring_invariants(S, late):
    for nk, niw in itertools.product(range(1, 17), (1, 2, 3, 4, 6)):
        if niw * max(S - 2, 0) > 63:
            continue
        check(S, nk, niw, late)


def test_checker_catches_a_short_wait():
    # a wait that lets this stage's own loads stay in flight must fail
    def bad_wait(S, nk, niw, it):
        return niw * (S - 1)
    global wait_count
    good = wait_count
    try:
        wait_count = bad_wait
        with pytest.raises(AssertionError):
            check(3, 6, 2, False)
    finally:
        wait_count = good


def test_checker_catches_an_early_refill():
    # refilling S stages ahead (into the slot being read) must fail
    def bad_schedule(S, nk, niw, late):
        ev = []
        for s in range(S):
            if s < nk:
                ev += [("issue", s, s % S)] * niw
        for it in range(nk):
            ev.append(("wait", 0, it))
            ev.append(("barrier", it))
            ev.append(("read", it, it % S))
            if it + S < nk:
                ev += [("issue", it + S, (it + S) % S)] * niw
        return ev
    global schedule
    good = schedule
    try:
        schedule = bad_schedule
        with pytest.raises(AssertionError):
            check(3, 6, 1, True)
    finally:
        schedule = good


def wait_count_by_iteration(S, nk, niw, it):
    # the NVFP4 form: S-2 stages are in flight behind stage it while
    # it < nk - (S - 2); one behind it at it == nk - 2 (S > 3); none after
    if S > 2 and it < nk - (S - 2):
        return niw * (S - 2)
    if S > 3 and it == nk - 2:
        return niw
    return 0


def slots_by_counters(S, nk):
    rd, wr, out = 0, S - 1, []
    for _ in range(nk):
        out.append((rd, wr))
        rd = 0 if rd == S - 1 else rd + 1
        wr = 0 if wr == S - 1 else wr + 1
    return out


@pytest.mark.parametrize("S", [2, 3, 4, 5])
def test_counter_form_matches_derived_form(S):
    for nk, niw in itertools.product(range(1, 40), (1, 2, 3)):
        for it in range(nk):
            assert wait_count_by_iteration(S, nk, niw, it) == wait_count(S, nk, niw, it), (S, nk, niw, it)
        assert slots_by_counters(S, nk) == [(it % S, (it + S - 1) % S) for it in range(nk)]
