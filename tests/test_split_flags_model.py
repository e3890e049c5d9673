"""Model of the split tail's flag protocol (CPU only), explored over every interleaving.

One published partial has a flag word, 0 when idle. The publisher, once its partial is
stored, swaps 0 -> epoch; if the swap fails (the owner gave up), it stores 0. The owner
polls up to N times for the epoch; if the polls run out it swaps 0 -> ABORT and counts
the wait as lost unless the swap found the epoch; after reading a partial it swaps
epoch -> 0. The invariants: the owner takes the partial only after this execute's
publisher stored it; the flag is 0 once both are done (lost wait or not); and so a
second execute with the same epoch (a replayed graph) behaves the same. A variant
without the ABORT marker (the owner clears the flag after a lost wait) is shown to
leave a stale flag behind."""
import itertools

import pytest

ABORT = -1
E = 7   # the epoch, the same in both executes (a replay)


def publisher():
    """Steps of the publisher: generator of actions on the shared state."""
    def p1(st):
        st["data"] = st["run"]        # the partial of this execute is stored before the flag
        if st["flag"] == 0:
            st["flag"] = E
            return "published"
        return "cas_failed"
    r = yield p1
    if r == "cas_failed":
        def p2(st):
            st["flag"] = 0
        yield p2


def owner(polls, abort_marker=True):
    got = None
    for _ in range(polls):
        def poll(st):
            return "seen" if st["flag"] == E else "not_yet"
        r = yield poll
        if r == "seen":
            got = True
            break
    if got is None:
        def giveup(st):
            if abort_marker:
                if st["flag"] == 0:
                    st["flag"] = ABORT
                    return "lost"
                return "seen" if st["flag"] == E else "lost"
            return "seen" if st["flag"] == E else "lost"
        r = yield giveup
        got = r == "seen"
    if got:
        def take(st):
            st["taken"] = st["data"]   # reads the partial
        yield take
        def clear(st):
            if st["flag"] == E:
                st["flag"] = 0
        yield clear
    else:
        def lost(st):
            st["lost"] += 1
            if not abort_marker:
                st["flag"] = 0         # the flawed variant: clear after giving up
        yield lost


def interleavings(a_len, b_len):
    for pos in itertools.combinations(range(a_len + b_len), a_len):
        yield [0 if i in pos else 1 for i in range(a_len + b_len)]


def run_one(st, polls, order, abort_marker=True):
    """Run one execute's publisher and owner with the scheduling `order` (0: publisher,
    1: owner; extra entries are ignored once a side is done)."""
    gens = [publisher(), owner(polls, abort_marker)]
    pending = [next(g) for g in gens]
    results = [None, None]
    st["taken"] = None
    for who in order:
        if pending[who] is None:
            continue
        res = pending[who](st)
        try:
            pending[who] = gens[who].send(res)
        except StopIteration:
            pending[who] = None
    for who in (0, 1):   # finish whatever is left, publisher first
        while pending[who] is not None:
            res = pending[who](st)
            try:
                pending[who] = gens[who].send(res)
            except StopIteration:
                pending[who] = None
    return st


def schedules(polls):
    n_owner = polls + 3
    for order in interleavings(2, n_owner):
        yield order


@pytest.mark.parametrize("polls", [0, 1, 2, 3])
def test_protocol_over_all_interleavings(polls):
    for o1 in schedules(polls):
        for o2 in schedules(polls):
            st = {"flag": 0, "data": None, "taken": None, "lost": 0}
            for run, order in ((1, o1), (2, o2)):
                st["run"] = run
                lost_before = st["lost"]
                run_one(st, polls, order)
                # the owner took this execute's partial, or counted a lost wait
                if st["lost"] == lost_before:
                    assert st["taken"] == run, (o1, o2, st)
                else:
                    assert st["taken"] is None
                # both done: the flag is idle again
                assert st["flag"] == 0, (o1, o2, st)


def test_without_the_abort_marker_a_stale_flag_survives():
    # owner gives up at once (no polls), clears the flag, then the late publisher sets it:
    # the next execute's owner, same epoch, would take a partial before it is stored
    st = {"flag": 0, "data": None, "taken": None, "lost": 0, "run": 1}
    run_one(st, 0, [1, 1, 1, 0, 0], abort_marker=False)
    assert st["lost"] == 1 and st["flag"] == E
    st["run"] = 2
    run_one(st, 1, [1, 1, 1, 1, 0, 0], abort_marker=False)   # owner polls before the publisher runs
    assert st["taken"] == 1   # the previous execute's partial: silently wrong
