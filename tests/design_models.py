"""Design proofs of the library's barrier kernels, by brute force over every
interleaving on tiny inputs.

The oracle's enumerator (oracle/enumerate.py) states the barrier of the
PTO-ISA SYNCALL guide, section 5.2, as the pages give it: one counter per
barrier and the plain per-round program WRITE, ARRIVE, POLL, READ.  The
kernels depart from that in three ways, none of which may change what is
computed, and this module models each of them on top of the plain
enumerator's round specifications so that the same exhaustive search checks
them:

  * striped counters -- each barrier's counter split into K stripes: member
    m arrives on stripe m mod K, derives its round from that stripe with the
    pages' rule, and is released once every stripe l holds epoch * n_l;
  * a two-level tree -- G group counters under one top counter: member m
    arrives on group m mod G; the arrival whose reply completes its group's
    round then arrives on the top counter (a separate atomic step, as in the
    kernel); every member polls the top counter for epoch * min(N, G);
  * pipelined schedules -- with ordering-only visibility the witness kernels
    write a member's witness `write_lead` of its own rounds ahead and may
    still read a row until `read_lag` rounds later.

Each check is the oracle's: every schedule terminates (no reachable state
with an unfinished participant and no enabled step), every READ of round r
sees each member's round-r write, and the final counts are the same in every
schedule.  Negative controls change one thing (poll with '==', skip a
barrier, a bad start value, a shallow ring) and must fail.

Test infrastructure: imported by tests only.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

from oracle.enumerate import (READ, WRITE, Result, RoundSpec, expected_final_counters,  # noqa: F401
                              grouped, whole_grid)

ARRIVE, TOP, POLL = 11, 12, 13


@dataclass(frozen=True)
class Striped:
    """K stripes per counter (K = 1: the pages' single counter)."""
    k: int

    def lines(self) -> int:
        return self.k


@dataclass(frozen=True)
class Tree:
    """G group counters and one top counter per barrier."""
    g: int

    def lines(self) -> int:
        return self.g + 1  # the top counter is line G


def _programs(rounds: Sequence[RoundSpec], n_participants: int, skip, write_lead: int,
              read_lag: int, tree: bool) -> List[List[Tuple[int, int]]]:
    """Per participant, its steps as (kind, round).  A barrier is ARRIVE,
    (TOP for a tree: a no-op unless that arrival completed its group), POLL.
    Plain order (write_lead = 0): WRITE, barrier, READ per member round.
    Pipelined (write_lead = a >= 1, read_lag = b >= 1), counted in the
    member's own rounds m_0, m_1, ...: the witnesses of m_0 .. m_{a-1} are
    written first, the witness of m_{i+a} right after passing the barrier of
    m_i, and the READ of m_i sits just before the arrival at m_{i+b} (the
    latest point the kernel may still be reading it; a slot that still
    holds m_i there held it since the barrier of m_i)."""
    skipped = set(skip)
    member_rounds: List[List[int]] = [[] for _ in range(n_participants)]
    for r, spec in enumerate(rounds):
        for p in spec.members:
            member_rounds[p].append(r)

    def barrier(p, r):
        if (p, r) in skipped:
            return []
        return [(ARRIVE, r)] + ([(TOP, r)] if tree else []) + [(POLL, r)]

    progs = []
    for p in range(n_participants):
        mine = member_rounds[p]
        steps: List[Tuple[int, int]] = []
        if write_lead <= 0:
            for r in mine:
                steps += [(WRITE, r)] + barrier(p, r) + [(READ, r)]
        else:
            a, b = write_lead, max(read_lag, 1)
            steps += [(WRITE, mine[j]) for j in range(min(a, len(mine)))]
            for i, r in enumerate(mine):
                if i - b >= 0:
                    steps.append((READ, mine[i - b]))
                steps += barrier(p, r)
                if i + a < len(mine):
                    steps.append((WRITE, mine[i + a]))
            steps += [(READ, mine[j]) for j in range(max(0, len(mine) - b), len(mine))]
        progs.append(steps)
    return progs


def explore(rounds: Sequence[RoundSpec], n_participants: int, *, layout=Striped(1),
            ring_depth: int = 4, poll_cmp: str = "ge",
            counter_init: Optional[Sequence[int]] = None, skip: Sequence[Tuple[int, int]] = (),
            write_lead: int = 0, read_lag: int = 0, max_states: int = 5_000_000) -> Result:
    """Every interleaving of the participants' steps under a counter layout.

    counter_init: a start value for line 0 of each barrier (stripe 0 or
    group 0).  Final counters are reported per barrier as the sum of its
    stripes or of its group counters (the number of member arrivals)."""
    tree = isinstance(layout, Tree)
    n_bar = 1 + max(spec.counter for spec in rounds)
    L = layout.lines()
    ctr0 = [0] * (n_bar * L)
    if counter_init is not None:
        for b, v in enumerate(counter_init):
            ctr0[b * L] = v
    progs = _programs(rounds, n_participants, skip, write_lead, read_lag, tree)
    res = Result()
    # state = (pcs, counters, epochs, completer flags, slots)
    start = ((0,) * n_participants, tuple(ctr0), (-1,) * n_participants,
             (False,) * n_participants, (-1,) * (ring_depth * n_participants))
    seen = set()
    stack = [start]
    while stack:
        state = stack.pop()
        if state in seen:
            continue
        seen.add(state)
        if len(seen) > max_states:
            raise RuntimeError("state space exceeds max_states")
        pcs, ctrs, eps, comp, slots = state
        successors = []
        all_done = True
        for p in range(n_participants):
            pc = pcs[p]
            if pc >= len(progs[p]):
                continue
            all_done = False
            kind, r = progs[p][pc]
            spec = rounds[r]
            base = spec.counter * L
            n = spec.n
            row = r % ring_depth
            nxt = _set(pcs, p, pc + 1)
            if kind == WRITE:
                successors.append((nxt, ctrs, eps, comp,
                                   _set(slots, row * n_participants + p, r)))
            elif kind == ARRIVE:
                if tree:
                    g = spec.members.index(p) % layout.g
                    ng = (n - g + layout.g - 1) // layout.g
                    line = base + g
                else:
                    k = layout.k
                    s = spec.members.index(p) % k
                    ng = (n - s + k - 1) // k
                    line = base + s
                before = ctrs[line]
                epoch = before // ng + 1     # the pages' rule on this line
                done = tree and before + 1 == epoch * ng  # a tree group's completer
                successors.append((nxt, _set(ctrs, line, before + 1), _set(eps, p, epoch),
                                   _set(comp, p, done), slots))
            elif kind == TOP:
                top = base + layout.g
                c2 = _set(ctrs, top, ctrs[top] + 1) if comp[p] else ctrs
                successors.append((nxt, c2, eps, _set(comp, p, False), slots))
            elif kind == POLL:
                epoch = eps[p]
                if tree:
                    want = [(base + layout.g, epoch * min(n, layout.g))]
                else:
                    k = layout.k
                    want = [(base + l, epoch * ((n - l + k - 1) // k)) for l in range(min(n, k))]
                ok = all((ctrs[i] >= w) if poll_cmp == "ge" else (ctrs[i] == w) for i, w in want)
                if ok:
                    successors.append((nxt, ctrs, eps, comp, slots))
            else:  # READ
                for q in spec.members:
                    got = slots[row * n_participants + q]
                    if got != r:
                        res.violations.append((r, p, q, got))
                successors.append((nxt, ctrs, eps, comp, slots))
        if all_done:
            member_lines = layout.g if tree else layout.k
            res.final_counters.add(tuple(sum(ctrs[b * L:b * L + member_lines])
                                         for b in range(n_bar)))
            res.complete_schedules_seen = True
            continue
        if not successors:
            res.deadlock = True
            if res.deadlock_state is None:
                res.deadlock_state = state
            continue
        stack.extend(successors)
    res.states = len(seen)
    return res


def _set(t: tuple, i: int, v) -> tuple:
    lst = list(t)
    lst[i] = v
    return tuple(lst)


# ---------------------------------------------------------------------------
# Full visibility with one L2 write-back per XCD.
#
# Here the model also has caches, because that is what the protocol is about.
# A member's WRITE lands in its XCD's L2 (every thread waits for its stores
# before arriving; the vector L1 is write-through).  Memory changes only
# when that XCD's leader writes the L2 back: every value the L2 holds for a
# slot goes to memory.  A READ after the acquire sees the L2 of its own XCD
# for a member of the same XCD, and memory for a member of another XCD (the
# acquire invalidates the reader's copies of lines it does not own).
#
# Per member round the program is WRITE, ARRIVE, POLL (striped, as above),
# then on the leader of each barrier's XCD (its first member there) LEAD
# (write back, then store the round in the XCD's flag), then FPOLL (every
# flag of an XCD with members of that barrier holds the round), then READ.
#
# Variants, each of which a check must catch:
#   "early_writeback"  the leader writes back and raises its flag right
#                      after its own arrival, before the round is complete
#   "no_writeback"     the leader raises its flag without writing back
#   "no_flag_poll"     members read right after the stripe poll
#   "own_flag_only"    members wait for their own XCD's flag alone
# ---------------------------------------------------------------------------
LEAD, FPOLL = 14, 15


def explore_xcd(rounds: Sequence[RoundSpec], n_participants: int, xcd_of: Sequence[int], *,
                k: int = 1, ring_depth: int = 4, variant: str = "ok",
                max_states: int = 5_000_000) -> Result:
    n_bar = 1 + max(spec.counter for spec in rounds)
    # leader of barrier b on XCD x: its first member there; XCDs with members
    leaders, xcds = {}, {}
    for spec in rounds:
        for p in spec.members:
            leaders.setdefault((spec.counter, xcd_of[p]), p)
            xcds.setdefault(spec.counter, set()).add(xcd_of[p])
    nx = 1 + max(xcd_of)
    progs = []
    for p in range(n_participants):
        steps: List[Tuple[int, int]] = []
        for r, spec in enumerate(rounds):
            if p not in spec.members:
                continue
            lead = leaders[(spec.counter, xcd_of[p])] == p
            steps += [(WRITE, r), (ARRIVE, r)]
            if lead and variant == "early_writeback":
                steps.append((LEAD, r))
            steps.append((POLL, r))
            if lead and variant != "early_writeback":
                steps.append((LEAD, r))
            if variant != "no_flag_poll":
                steps.append((FPOLL, r))
            steps.append((READ, r))
        progs.append(steps)
    n_slots = ring_depth * n_participants
    res = Result()
    # state = (pcs, counters, epochs, flags, l2 per XCD, memory)
    start = ((0,) * n_participants, (0,) * (n_bar * k), (-1,) * n_participants,
             (0,) * (n_bar * nx), ((-1,) * n_slots,) * nx, (-1,) * n_slots)
    seen = set()
    stack = [start]
    while stack:
        state = stack.pop()
        if state in seen:
            continue
        seen.add(state)
        if len(seen) > max_states:
            raise RuntimeError("state space exceeds max_states")
        pcs, ctrs, eps, flags, l2, mem = state
        successors = []
        all_done = True
        for p in range(n_participants):
            pc = pcs[p]
            if pc >= len(progs[p]):
                continue
            all_done = False
            kind, r = progs[p][pc]
            spec = rounds[r]
            b, n, x = spec.counter, spec.n, xcd_of[p]
            nxt = _set(pcs, p, pc + 1)
            slot = (r % ring_depth) * n_participants
            if kind == WRITE:
                successors.append((nxt, ctrs, eps, flags,
                                   _set(l2, x, _set(l2[x], slot + p, r)), mem))
            elif kind == ARRIVE:
                s = spec.members.index(p) % k
                ns = (n - s + k - 1) // k
                before = ctrs[b * k + s]
                successors.append((nxt, _set(ctrs, b * k + s, before + 1),
                                   _set(eps, p, before // ns + 1), flags, l2, mem))
            elif kind == POLL:
                e = eps[p]
                if all(ctrs[b * k + l] >= e * ((n - l + k - 1) // k) for l in range(min(n, k))):
                    successors.append((nxt, ctrs, eps, flags, l2, mem))
            elif kind == LEAD:
                m = mem
                if variant != "no_writeback":
                    m = tuple(v if v >= 0 else mv for v, mv in zip(l2[x], mem))
                successors.append((nxt, ctrs, eps, _set(flags, b * nx + x, eps[p]), l2, m))
            elif kind == FPOLL:
                watched = [x] if variant == "own_flag_only" else xcds[b]
                if all(flags[b * nx + y] >= eps[p] for y in watched):
                    successors.append((nxt, ctrs, eps, flags, l2, mem))
            else:  # READ
                for q in spec.members:
                    got = l2[x][slot + q] if xcd_of[q] == x else mem[slot + q]
                    if got != r:
                        res.violations.append((r, p, q, got))
                successors.append((nxt, ctrs, eps, flags, l2, mem))
        if all_done:
            res.final_counters.add(tuple(sum(ctrs[bb * k:(bb + 1) * k]) for bb in range(n_bar)))
            res.complete_schedules_seen = True
            continue
        if not successors:
            res.deadlock = True
            if res.deadlock_state is None:
                res.deadlock_state = state
            continue
        stack.extend(successors)
    res.states = len(seen)
    return res
