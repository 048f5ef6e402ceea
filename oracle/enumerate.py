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
              skip: Sequence[Tuple[int, int]] = (),
              early_write: bool = False, write_lead: int = 0,
              read_lag: int = 0) -> List[List[Tuple[int, int]]]:
    """Per participant: the flat list of (step kind, round) it executes.

    In the plain schedule every member round is WRITE, ARRIVE, POLL, READ.
    A pipelined schedule (write_lead = a >= 1) counts in the participant's
    own member rounds m_0, m_1, ...: the witnesses of m_0 .. m_{a-1} are
    written before the first barrier, the witness of m_{i+a} right after
    passing the barrier of m_i, and the read of m_i may still be in flight
    until the participant arrives at m_{i+b} (b = read_lag >= 1).  The READ
    step sits at that latest point: a slot that still holds round m_i there
    held it since the barrier of m_i (a slot is only ever overwritten by a
    later round), so this placement covers every earlier one.  early_write
    is a = b = 1.  A skipped barrier drops that round's ARRIVE and POLL."""
    if early_write:
        write_lead, read_lag = max(write_lead, 1), max(read_lag, 1)
    skipped = set(skip)
    member_rounds: List[List[int]] = [[] for _ in range(n_participants)]
    for r, spec in enumerate(rounds):
        for p in spec.members:
            member_rounds[p].append(r)
    progs: List[List[Tuple[int, int]]] = []
    for p in range(n_participants):
        mine = member_rounds[p]
        steps: List[Tuple[int, int]] = []
        if write_lead <= 0:
            for r in mine:
                steps.append((WRITE, r))
                if (p, r) not in skipped:
                    steps.append((ARRIVE, r))
                    steps.append((POLL, r))
                steps.append((READ, r))
        else:
            a, b = write_lead, max(read_lag, 1)
            steps.extend((WRITE, mine[j]) for j in range(min(a, len(mine))))
            for i, r in enumerate(mine):
                if i - b >= 0:
                    steps.append((READ, mine[i - b]))
                if (p, r) not in skipped:
                    steps.append((ARRIVE, r))
                    steps.append((POLL, r))
                if i + a < len(mine):
                    steps.append((WRITE, mine[i + a]))
            steps.extend((READ, mine[j]) for j in range(max(0, len(mine) - b), len(mine)))
        progs.append(steps)
    return progs


def enumerate_schedules(rounds: Sequence[RoundSpec], n_participants: int, *,
                        ring_depth: int = 4, poll_cmp: str = "ge",
                        counter_init: Optional[Sequence[int]] = None,
                        skip: Sequence[Tuple[int, int]] = (),
                        early_write: bool = False, stripes: int = 1,
                        write_lead: int = 0, read_lag: int = 0,
                        max_states: int = 5_000_000) -> Result:
    """Explore every interleaving of the participants' steps.

    rounds        the global round list (RoundSpec per round)
    ring_depth    D, the number of witness slot rows reused round-robin
    poll_cmp      'ge' (counter >= target) or 'eq' (counter == target)
    counter_init  starting value of each counter (default all zero)
    skip          (participant, round) pairs whose barrier is left out
                  (the participant still writes and reads)
    early_write   the pipelined step order with a = b = 1 (see _programs)
    write_lead    a, read_lag b: a pipelined step order (see _programs)
    stripes       K: each counter is split into K stripes; the member with
                  index m in its round's member list arrives on stripe m mod K,
                  whose member count is n_s = ceil((N - s) / K), derives its
                  round e = before // n_s + 1 from that stripe, and is released
                  once every stripe l < min(N, K) holds at least e * n_l.  K = 1
                  is the single counter of the SYNCALL guide.
    """
    n_counters = 1 + max(spec.counter for spec in rounds)
    K = stripes
    ctr0 = (tuple(c for c in counter_init for _ in range(1)) if counter_init is not None
            else (0,) * n_counters)
    if counter_init is not None:
        # an initial value applies to stripe 0 of each counter
        ctr0 = tuple(v if s == 0 else 0 for v in counter_init for s in range(K))
    else:
        ctr0 = (0,) * (n_counters * K)
    progs = _programs(rounds, n_participants, skip, early_write, write_lead, read_lag)
    res = Result()

    # state = (pcs, counters, targets, slots)
    #   pcs[p]     = index of participant p's next step
    #   targets[p] = the round (epoch) derived at its last ARRIVE (or -1)
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
                st = spec.members.index(p) % K
                ns = (n - st + K - 1) // K
                before = ctrs[g * K + st]
                epoch = before // ns + 1       # target = epoch * ns, the pages' rule per stripe
                successors.append((nxt, _set(ctrs, g * K + st, before + 1), _set(tgts, p, epoch),
                                   slots))
            elif kind == POLL:
                n = spec.n
                epoch = tgts[p]
                ok = True
                for lane in range(min(n, K)):
                    nl = (n - lane + K - 1) // K
                    c = ctrs[g * K + lane]
                    ok = ok and (c >= epoch * nl if poll_cmp == "ge" else c == epoch * nl)
                if ok:
                    successors.append((nxt, ctrs, tgts, slots))
            else:  # READ
                for q in spec.members:
                    got = slots[row * n_participants + q]
                    if got != r:
                        res.violations.append((r, p, q, got))
                successors.append((nxt, ctrs, tgts, slots))
        if all_done:
            res.final_counters.add(tuple(sum(ctrs[g * K:(g + 1) * K]) for g in range(n_counters)))
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
