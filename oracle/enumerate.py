"""Brute-force enumeration of every arrival order of the soft epoch barrier.

TEST INFRASTRUCTURE ONLY: part of the oracle.  Nothing in the product path
may import it.

Sources (cited by page title and section):
  [SYNCALL] "PTO-ISA 跨核同步屏障 SYNCALL 实战指南" (PTO-ISA SYNCALL guide):
    §2   the barrier is an arrival relation over the current participant set;
    §4.1 the counter must start at zero;
    §4.2 usedCores picks the participant count, non-members never call;
    §5.2 Soft mode: atomic +1 returning the old value, target derived from it,
         poll until the counter reaches the target;
    §6.1 the test pattern of flag slots written before and read after;
    §6.2 every participant enters the same barriers in the same order the
         same number of times, otherwise rounds slip and the barrier hangs.

Model.  Each participant runs a fixed program: for every round it belongs to
it performs four atomic steps in order

    WRITE   slot[r mod D][p] := r            (its witness for round r)
    ARRIVE  before := ctr[g]; ctr[g] += 1; target := (before // N + 1) * N
    POLL    enabled only while the release condition holds
    READ    reads slot[r mod D][q] for every member q of round r

where g is the round's counter and N its participant count.  A depth-first
search over every interleaving (memoised on the full state) checks that

  * every schedule terminates -- no reachable state has an unfinished
    participant while no step is enabled (that state is a deadlock);
  * at every READ of round r, each member's slot holds its round-r write
    (so every round-r write precedes every round-r read, and no later write
    has overwritten it);
  * the final counters are the same in every schedule.

READ is one atomic step.  That loses no violation: another participant's
write is enabled independently of how far a reader has got through its
reads, so a schedule that slips the write between two reads has a twin that
puts it before the whole READ.

Negative controls are built from the same model by changing one thing:
poll with '==' instead of '>=', drop one participant's barrier, declare more
participants than call, start the counter at a value that is not a multiple
of N, or shrink the slot ring.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

WRITE, ARRIVE, POLL, READ = 0, 1, 2, 3


@dataclass(frozen=True)
class RoundSpec:
    """One round of the schedule: which counter it uses and who takes part."""

    counter: int
    members: Tuple[int, ...]
    declared_n: Optional[int] = None  # participant count passed to the barrier

    @property
    def n(self) -> int:
        return self.declared_n if self.declared_n is not None else len(self.members)


@dataclass
class Result:
    deadlock: bool = False
    deadlock_state: Optional[tuple] = None
    violations: List[tuple] = field(default_factory=list)
    final_counters: set = field(default_factory=set)
    states: int = 0
    complete_schedules_seen: bool = False


def _programs(rounds: Sequence[RoundSpec], n_participants: int,
              skip: Sequence[Tuple[int, int]] = ()) -> List[List[Tuple[int, int]]]:
    """Per participant: the flat list of (step kind, round) it executes --
    WRITE, ARRIVE, POLL, READ for every round it belongs to.  A skipped
    barrier drops that round's ARRIVE and POLL (the participant still writes
    and reads)."""
    skipped = set(skip)
    progs: List[List[Tuple[int, int]]] = []
    for p in range(n_participants):
        steps: List[Tuple[int, int]] = []
        for r, spec in enumerate(rounds):
            if p not in spec.members:
                continue
            steps.append((WRITE, r))
            if (p, r) not in skipped:
                steps.append((ARRIVE, r))
                steps.append((POLL, r))
            steps.append((READ, r))
        progs.append(steps)
    return progs


def enumerate_schedules(rounds: Sequence[RoundSpec], n_participants: int, *,
                        ring_depth: int = 4, poll_cmp: str = "ge",
                        counter_init: Optional[Sequence[int]] = None,
                        skip: Sequence[Tuple[int, int]] = (),
                        max_states: int = 5_000_000) -> Result:
    """Explore every interleaving of the participants' steps.

    rounds        the global round list (RoundSpec per round)
    ring_depth    D, the number of witness slot rows reused round-robin
    poll_cmp      'ge' (counter >= target) or 'eq' (counter == target)
    counter_init  starting value of each counter (default all zero)
    skip          (participant, round) pairs whose barrier is left out
                  (the participant still writes and reads)
    """
    n_counters = 1 + max(spec.counter for spec in rounds)
    ctr0 = tuple(counter_init) if counter_init is not None else (0,) * n_counters
    progs = _programs(rounds, n_participants, skip)
    res = Result()

    # state = (pcs, counters, targets, slots)
    #   pcs[p]     = index of participant p's next step
    #   targets[p] = the target derived at its last ARRIVE (or -1)
    #   slots      = tuple over (ring row, participant) of the last round written
    start = ((0,) * n_participants, ctr0, (-1,) * n_participants,
             (-1,) * (ring_depth * n_participants))
    seen = set()
    stack = [start]
    while stack:
        state = stack.pop()
        if state in seen:
            continue
        seen.add(state)
        if len(seen) > max_states:
            raise RuntimeError("state space exceeds max_states")
        pcs, ctrs, tgts, slots = state
        successors = []
        all_done = True
        for p in range(n_participants):
            pc = pcs[p]
            if pc >= len(progs[p]):
                continue
            all_done = False
            kind, r = progs[p][pc]
            spec = rounds[r]
            g = spec.counter
            row = r % ring_depth
            nxt = _set(pcs, p, pc + 1)
            if kind == WRITE:
                new_slots = list(slots)
                new_slots[row * n_participants + p] = r
                successors.append((nxt, ctrs, tgts, tuple(new_slots)))
            elif kind == ARRIVE:
                n = spec.n
                before = ctrs[g]
                target = (before // n + 1) * n     # the pages' rule
                successors.append((nxt, _set(ctrs, g, before + 1), _set(tgts, p, target), slots))
            elif kind == POLL:
                c = ctrs[g]
                if (c >= tgts[p]) if poll_cmp == "ge" else (c == tgts[p]):
                    successors.append((nxt, ctrs, tgts, slots))
            else:  # READ
                for q in spec.members:
                    got = slots[row * n_participants + q]
                    if got != r:
                        res.violations.append((r, p, q, got))
                successors.append((nxt, ctrs, tgts, slots))
        if all_done:
            res.final_counters.add(tuple(ctrs))
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
# Schedules used by the tests.
# ---------------------------------------------------------------------------

def whole_grid(n_participants: int, n_rounds: int, used_cores: int = 0,
               n_members: Optional[int] = None) -> List[RoundSpec]:
    """Every round on counter 0.  Members are ids 0..n_members-1 (default all);
    the barrier is told N = used_cores (0 = the member count)."""
    m = n_participants if n_members is None else n_members
    members = tuple(range(m))
    declared = used_cores if used_cores != 0 else None
    return [RoundSpec(0, members, declared) for _ in range(n_rounds)]


def grouped(n_participants: int, n_rounds: int) -> List[RoundSpec]:
    """Round r: r mod 3 == 0 -> group A (even ids, counter 0); 1 -> group B
    (odd ids, counter 1); 2 -> everyone (counter 2)."""
    even = tuple(p for p in range(n_participants) if p % 2 == 0)
    odd = tuple(p for p in range(n_participants) if p % 2 == 1)
    allp = tuple(range(n_participants))
    out = []
    for r in range(n_rounds):
        kind = r % 3
        out.append(RoundSpec(kind, even if kind == 0 else odd if kind == 1 else allp))
    return out


def expected_final_counters(rounds: Sequence[RoundSpec]) -> Tuple[int, ...]:
    """Final value of each counter when every member arrives once per round."""
    n_counters = 1 + max(spec.counter for spec in rounds)
    totals = [0] * n_counters
    for spec in rounds:
        totals[spec.counter] += len(spec.members)
    return tuple(totals)


def summarize(res: Result) -> Dict[str, object]:
    return {
        "deadlock": res.deadlock,
        "violations": len(res.violations),
        "final_counters": sorted(res.final_counters),
        "states": res.states,
    }
