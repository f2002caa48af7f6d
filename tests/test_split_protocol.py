"""Model check of the K-split hand-off protocol of the chunked GEMM (the
workgroup pair that splits one tile's K loop; the device code is
split_exchange and the start ticket in csrc/mc2_gemm.hip).

The two halves are modelled as step machines over the shared control words
(ctl0: start tickets, F[x]: "half x has written its slot") and the two partial
slots, and every interleaving of their steps is explored, including those in
which one half runs to its end before the other starts. For both policies
(PAIR: the first half waits for a running partner; ALONE: it never waits) the
checks are:
  - no interleaving deadlocks, and a half only ever waits for a half that has
    taken its start ticket (so it waits for a running workgroup only);
  - each of the tile's two row halves is finalized exactly once, with the
    value P0 + P1 (the partials of both K halves for those rows);
  - the control words are all zero at the end (the next call starts clean).
A planted mistake (the late half forgetting to reset ctl0, or the early half
not re-checking whether its partner started) must make the check fail.
"""
import itertools

import pytest

PAIR, ALONE = 0, 1


class Half:
    """One K half h of a tile pair, stepping through the protocol."""

    def __init__(self, h, policy, bug=None):
        self.h, self.policy, self.bug = h, policy, bug
        self.pc = 0
        self.ticket = None
        self.alone = None
        self.done = False
        self.waiting = False
        # partial of this half for row halves 0 and 1 (symbolic: (K half, rows))
        self.acc = {0: {(h, 0)}, 1: {(h, 1)}}
        self.final = {}

    def early(self):
        return self.ticket == 0


def step(u, st):
    """Executes one step of half u on shared state st; returns False if u is
    blocked (waiting on a mark not yet set)."""
    h = u.h
    if u.pc == 0:  # start ticket
        u.ticket = st["ctl0"]
        st["ctl0"] += 1
        st["started"][h] = True
        u.pc = 10 if u.ticket == 0 and u.policy == ALONE else 1
        return True
    if u.pc == 10:  # policy ALONE: the early half's separate compare-and-swap 1 -> 3
        if st["ctl0"] == 1:
            st["ctl0"] = 3
        u.pc = 1
        return True
    if u.pc == 1:  # end of the K loop: the early half's decision
        if u.early():
            e = st["ctl0"]
            if e == 1 and u.bug != "no_recheck":
                st["ctl0"] = 3
            u.alone = (e != 2) if u.bug != "no_recheck" else True
        else:
            u.alone = u.ticket != 1
        u.pc = 2
        return True
    if u.pc == 2:  # the partial stores (complete before the mark)
        # slot x holds row half 1 - x; a wave of row half rh writes slot 1 - rh
        for rh in (0, 1):
            sends = (u.alone or rh != h) if u.early() else (not u.alone and rh != h)
            if sends:
                st["slot"][1 - rh] = set(u.acc[rh])
        u.pc = 3
        return True
    if u.pc == 3:  # the mark, or the early half leaving alone
        if u.early() or not u.alone:
            st["F"][h] = 1
        if u.early() and u.alone:
            u.done = True
            u.pc = 99
            return True
        u.pc = 4
        return True
    if u.pc == 4:  # wait for the partner's mark
        if st["F"][1 - h] == 0:
            u.waiting = True
            return False
        u.waiting = False
        u.pc = 5
        return True
    if u.pc == 5:  # add the partner's part of the rows this half finalizes
        for rh in (0, 1):
            if u.alone or rh == h:
                u.acc[rh] = u.acc[rh] | st["slot"][1 - rh]
        u.pc = 6
        return True
    if u.pc == 6:  # reset the partner's mark (and, the late half, the tickets)
        st["F"][1 - h] = 0
        if not u.early() and u.bug != "no_reset":
            st["ctl0"] = 0
        u.pc = 7
        return True
    if u.pc == 7:  # finalize
        for rh in ((0, 1) if u.alone else (h,)):
            st["final"].setdefault(rh, []).append(frozenset(u.acc[rh]))
        u.done = True
        u.pc = 99
        return True
    raise AssertionError(u.pc)


def explore(policy, bug=None):
    """All interleavings of the two halves; returns (#terminal states, problems)."""
    problems = []
    terminals = 0

    def dfs(a, b, st):
        nonlocal terminals
        if a.done and b.done:
            terminals += 1
            want = {0: frozenset({(0, 0), (1, 0)}), 1: frozenset({(0, 1), (1, 1)})}
            for rh in (0, 1):
                got = st["final"].get(rh, [])
                if got != [want[rh]]:
                    problems.append(f"row half {rh} finalized as {got}")
            if st["ctl0"] != 0 or st["F"] != [0, 0]:
                problems.append(f"control words left {st['ctl0']}, {st['F']}")
            return
        moved = False
        for i, u in enumerate((a, b)):
            if u.done:
                continue
            ua, ub = clone(a), clone(b)
            s2 = clone_state(st)
            uu = (ua, ub)[i]
            if step(uu, s2):
                moved = True
                dfs(ua, ub, s2)
            elif not s2["started"][1 - uu.h]:
                problems.append(f"half {uu.h} waits for a half that has not started")
        if not moved:
            problems.append("deadlock")

    st = {"ctl0": 0, "F": [0, 0], "slot": {0: set(), 1: set()}, "final": {},
          "started": [False, False]}
    dfs(Half(0, policy, bug), Half(1, policy, bug), st)
    return terminals, problems


def clone(u):
    v = Half.__new__(Half)
    v.__dict__ = {k: (dict((kk, set(vv)) for kk, vv in val.items()) if k == "acc" else
                      dict(val) if isinstance(val, dict) else val)
                  for k, val in u.__dict__.items()}
    return v


def clone_state(st):
    return {"ctl0": st["ctl0"], "F": list(st["F"]),
            "slot": {k: set(v) for k, v in st["slot"].items()},
            "final": {k: list(v) for k, v in st["final"].items()},
            "started": list(st["started"])}


@pytest.mark.parametrize("policy", [PAIR, ALONE])
def test_protocol_every_interleaving(policy):
    terminals, problems = explore(policy)
    assert terminals > 0
    assert not problems, sorted(set(problems))[:5]


def test_both_modes_are_reached():
    """Under PAIR some interleavings end in the pair exchange (each half
    finalizes one row half) and some in the hand-over (one finalizes both)."""
    modes = set()

    def run(order):
        a, b = Half(0, PAIR), Half(1, PAIR)
        st = {"ctl0": 0, "F": [0, 0], "slot": {0: set(), 1: set()}, "final": {},
              "started": [False, False]}
        for who in order:
            u = (a, b)[who]
            if not u.done:
                step(u, st)
        while not (a.done and b.done):  # finish whatever is left
            progressed = False
            for u in (a, b):
                if not u.done and step(u, st):
                    progressed = True
            assert progressed
        modes.add((a.alone, b.alone))

    for order in itertools.product((0, 1), repeat=6):
        run(order)
    assert (False, False) in modes  # pair exchange
    assert any(m in modes for m in ((True, True),))  # hand-over


@pytest.mark.parametrize("bug", ["no_reset", "no_recheck"])
def test_planted_mistakes_are_caught(bug):
    _, problems = explore(PAIR, bug)
    assert problems
