"""Pins for the barrier half of the oracle (CPU only).

The round simulator in oracle/ccb_oracle.c is checked against things that do
not come from it: brute-force enumeration of every arrival order, closed forms
for the witness sums and final counters, SplitMix64's published outputs, and
the constants printed on the SYNCALL page (tests/golden/syncall_constants.txt).
"""

import os

import numpy as np
import pytest

import oracle
from oracle import enumerate as en

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
M64 = (1 << 64) - 1


def _golden_constants():
    out = {}
    with open(os.path.join(GOLDEN, "syncall_constants.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = int(v)
    return out


# --- SplitMix64 -------------------------------------------------------------
# Published output sequences of SplitMix64 (Steele, Lea & Flood, OOPSLA 2014),
# as widely reproduced for the generator: the first three outputs for seed 0
# and for seed 1234567.
SPLITMIX_SEED0 = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
SPLITMIX_SEED1234567 = [6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_splitmix64_published_sequences():
    for n, want in enumerate(SPLITMIX_SEED0, start=1):
        assert oracle.splitmix64_nth(0, n) == want
    for n, want in enumerate(SPLITMIX_SEED1234567, start=1):
        assert oracle.splitmix64_nth(1234567, n) == want


def test_splitmix64_shift_invariance():
    # Advancing the seed by one gamma shifts the sequence by one output.
    g = 0x9E3779B97F4A7C15
    for seed in (0, 1, 99, 2**63 + 5):
        for n in (1, 2, 7, 2**40 + 3):
            assert oracle.splitmix64_nth(seed, n + 1) == oracle.splitmix64_nth((seed + g) & M64, n)


def test_witness_hash_keying():
    # hash(seed, r, w) = high half of output number r*2^32 + w + 1.
    assert oracle.witness_hash(0, 0, 0) == SPLITMIX_SEED0[0] >> 32
    assert oracle.witness_hash(0, 0, 1) == SPLITMIX_SEED0[1] >> 32
    assert oracle.witness_hash(0, 0, 2) == SPLITMIX_SEED0[2] >> 32
    assert oracle.witness_hash(1234567, 0, 1) == SPLITMIX_SEED1234567[1] >> 32
    for seed, r, w in [(1, 5, 7), (4, 99_999, 511), (3, 1, 0)]:
        n = (r << 32) + w + 1
        assert oracle.witness_hash(seed, r, w) == oracle.splitmix64_nth(seed, n) >> 32


# --- epoch target and participant count --------------------------------------

def test_epoch_target_is_next_multiple():
    # SYNCALL guide §5.2: the release point is the count once the last member
    # of the current round has arrived -- the smallest multiple of N above the
    # old value.  Found here by search, not by the formula.
    for n in range(1, 10):
        for before in range(0, 200):
            t = before + 1
            while t % n != 0:
                t += 1
            assert oracle.epoch_target(before, n) == t, (before, n)


def test_epoch_target_checked_at_the_int32_limit():
    # SYNCALL guide §4.1 types the counter int32: a target above 2^31 - 1 can
    # never be reached, an old value below zero is a wrapped counter.  The
    # next multiple is found by search on Python integers, then compared
    # with the limit.
    limit = 2**31 - 1
    for n in (1, 2, 3, 4, 7, 64, 1000, 65_537):
        top = limit - limit % n          # largest multiple of n in range
        for before in (0, n - 1, top - n - 1, top - n, top - 1, top, limit):
            t = before + 1
            while t % n != 0:
                t += 1
            rc, got = oracle.epoch_target_checked(before, n)
            if t <= limit:
                assert (rc, got) == (oracle.OK, t), (before, n)
            else:
                assert rc == oracle.INVALID_VALUE, (before, n)
    assert oracle.epoch_target_checked(-1, 4)[0] == oracle.INVALID_VALUE
    assert oracle.epoch_target_checked(-(2**31), 1)[0] == oracle.INVALID_VALUE


def test_round_simulator_stops_at_the_int32_limit():
    # 8 members from one round below the limit: one more round completes and
    # reaches the largest multiple of 8 in range; a second cannot.
    top = (2**31 - 1) // 8 * 8
    _, _, ctr, rc = oracle.slot_rounds(0, 1, 8, 0, counter0=top - 8)
    assert (rc, ctr) == (oracle.OK, top)
    _, _, _, rc = oracle.slot_rounds(0, 2, 8, 0, counter0=top - 8)
    assert rc == oracle.INVALID_VALUE


def test_participants_rule():
    assert oracle.participants(0, 256) == 256
    assert oracle.participants(128, 256) == 128
    assert oracle.participants(256, 256) == 256
    assert oracle.participants(-1, 256) == -1
    assert oracle.participants(257, 256) == -1


def test_mix_participants_rule():
    # SYNCALL guide §4.2: Mix count = blocks x (1 + ratio); the ratios the
    # pages' Mix tests use and the default ratio come from the golden file.
    g = _golden_constants()
    for ratio in (g["mix_test_ratio_a"], g["mix_test_ratio_b"], g["mix_default_aiv_ratio"]):
        for groups in (1, 3, 8):
            assert oracle.mix_participants(groups, ratio, 64) == groups + groups * ratio
        assert oracle.mix_participants(0, ratio, 48) == 48          # whole launch
        assert oracle.mix_participants(64, ratio, 64) == -1         # more than launched
    assert oracle.mix_participants(-1, 1, 8) == -1
    assert oracle.mix_participants(1, -1, 8) == -1


def test_golden_constants_present():
    c = _golden_constants()
    assert c["soft_max_poll_iterations"] == 1_000_000
    assert c["soft_workspace_int32"] * 4 == 64
    assert c["idle_core_mark"] == 2
    assert c["counter_initial"] == 0


# --- brute-force enumeration -------------------------------------------------

@pytest.mark.parametrize("p,r", [(1, 3), (2, 1), (2, 2), (2, 3), (3, 1), (3, 2), (3, 3)])
def test_enumerator_whole_grid(p, r):
    rounds = en.whole_grid(p, r)
    res = en.enumerate_schedules(rounds, p)
    assert not res.deadlock
    assert res.violations == []
    assert res.final_counters == {(r * p,)}


def test_enumerator_partial_participation():
    # 3 launched, usedCores = 2: members 0 and 1, participant 2 never calls.
    rounds = en.whole_grid(3, 3, used_cores=2, n_members=2)
    res = en.enumerate_schedules(rounds, 3)
    assert not res.deadlock and res.violations == []
    assert res.final_counters == {(6,)}


def test_enumerator_grouped_depth4_safe():
    rounds = en.grouped(4, 6)
    res = en.enumerate_schedules(rounds, 4, ring_depth=4)
    assert not res.deadlock
    assert res.violations == []
    assert res.final_counters == {en.expected_final_counters(rounds)} == {(4, 4, 8)}


def test_enumerator_grouped_depth3_violates():
    # A B member can finish the mix round, pass the next B round without any A
    # member and write its next mix-round slot while an A member still reads
    # the previous mix round: a ring of 3 rows is not enough for this pattern.
    rounds = en.grouped(4, 6)
    res = en.enumerate_schedules(rounds, 4, ring_depth=3)
    assert not res.deadlock
    assert res.violations != []


def test_enumerator_whole_grid_depth2_safe_depth1_violates():
    rounds = en.whole_grid(3, 3)
    assert en.enumerate_schedules(rounds, 3, ring_depth=2).violations == []
    assert en.enumerate_schedules(rounds, 3, ring_depth=1).violations != []


# --- negative controls --------------------------------------------------------

def test_poll_with_equality_deadlocks():
    # A fast member can arrive for the next round before a slow member's next
    # poll, so the counter overshoots the slow member's target: '==' hangs.
    res = en.enumerate_schedules(en.whole_grid(2, 2), 2, poll_cmp="eq")
    assert res.deadlock
    res_ge = en.enumerate_schedules(en.whole_grid(2, 2), 2, poll_cmp="ge")
    assert not res_ge.deadlock


def test_skipped_barrier_deadlocks():
    # SYNCALL guide §6.2: entering a barrier one time fewer slips the rounds.
    res = en.enumerate_schedules(en.whole_grid(2, 3), 2, skip=[(0, 1)])
    assert res.deadlock


def test_used_cores_above_callers_deadlocks():
    # SYNCALL guide §6.3: a participant count that does not match who calls hangs.
    rounds = en.whole_grid(2, 1, used_cores=3, n_members=2)
    res = en.enumerate_schedules(rounds, 2)
    assert res.deadlock


def test_nonzero_start_breaks_witness():
    # SYNCALL guide §4.1: a counter that is not zeroed miscounts; a start that
    # is not a multiple of N releases a round early.
    res = en.enumerate_schedules(en.whole_grid(2, 2), 2, counter_init=[1])
    assert res.violations != []


def test_multiple_of_n_start_is_harmless():
    res = en.enumerate_schedules(en.whole_grid(2, 2), 2, counter_init=[4])
    assert not res.deadlock and res.violations == []
    assert res.final_counters == {(8,)}


# --- round simulator vs closed forms ----------------------------------------

def _hash_py(seed, r, w):
    state = (seed + 0x9E3779B97F4A7C15 * (((r << 32) | w) + 1)) & M64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return (z ^ (z >> 31)) >> 32


def _closed_form(seed, rounds, n_grid, member_sets):
    out = np.zeros((rounds, n_grid), dtype=np.uint32)
    for r in range(rounds):
        members = member_sets(r)
        s = sum(_hash_py(seed, r, q) for q in members) & 0xFFFFFFFF
        for w in members:
            out[r, w] = s
    return out


def test_slot_rounds_small_workload_closed_form():
    # 8 workgroups, 100 rounds, seed 0; final counter 8 * 100 = 800.
    out, status, ctr, rc = oracle.slot_rounds(0, 100, 8)
    assert rc == 0 and ctr == 800
    assert (status == 1).all()
    np.testing.assert_array_equal(out, _closed_form(0, 100, 8, lambda r: range(8)))


def test_slot_rounds_partial_closed_form():
    out, status, ctr, rc = oracle.slot_rounds(1, 40, 256, 128)
    assert rc == 0 and ctr == 40 * 128
    assert (status[:128] == 1).all() and (status[128:] == 2).all()
    np.testing.assert_array_equal(out, _closed_form(1, 40, 256, lambda r: range(128)))
    assert (out[:, 128:] == 0).all()


def test_slot_rounds_grid_final_counters():
    # 256 workgroups x 10,000 rounds, then 128 of them.
    _, _, ctr, rc = oracle.slot_rounds(1, 10_000, 256, 0)
    assert rc == 0 and ctr == 2_560_000
    _, _, ctr, rc = oracle.slot_rounds(1, 10_000, 256, 128)
    assert rc == 0 and ctr == 1_280_000


def test_slot_rounds_invalid_counts():
    assert oracle.slot_rounds(0, 1, 8, -1)[3] == oracle.INVALID_VALUE
    assert oracle.slot_rounds(0, 1, 8, 9)[3] == oracle.INVALID_VALUE


def test_slot_rounds_bad_start_detected():
    # Start not a multiple of N: the sequential schedule finds a member whose
    # target runs past the round's arrivals.
    _, _, _, rc = oracle.slot_rounds(0, 3, 4, 0, counter0=1)
    assert rc == oracle.DEADLOCK
    _, _, ctr, rc = oracle.slot_rounds(0, 3, 4, 0, counter0=8)
    assert rc == 0 and ctr == 8 + 12


def test_grouped_rounds_closed_form_small():
    n = 16
    out, status, ctrs, rc = oracle.grouped_rounds(4, 30, n)
    assert rc == 0
    assert ctrs == (10 * 8, 10 * 8, 10 * 16)
    sets = {0: range(0, n, 2), 1: range(1, n, 2), 2: range(n)}
    np.testing.assert_array_equal(out, _closed_form(4, 30, n, lambda r: sets[r % 3]))


def test_grouped_rounds_final_counters_closed_form():
    # 512 workgroups; 3,001 rounds -> 1,001 A, 1,000 B, 1,000 mix rounds.
    _, _, ctrs, rc = oracle.grouped_rounds(4, 3001, 512)
    assert rc == 0
    assert ctrs == (1001 * 256, 1000 * 256, 1000 * 512)


def test_grouped_full_counters_formula():
    # 100,000 rounds: 33,334 A, 33,333 B, 33,333 mix rounds (checked on the
    # round pattern alone; the full simulation runs in the GPU parity test).
    kinds = np.arange(100_000) % 3
    assert (int((kinds == 0).sum()) * 256, int((kinds == 1).sum()) * 256,
            int((kinds == 2).sum()) * 512) == (8_533_504, 8_533_248, 17_066_496)


# The method on real host threads: T threads write, pass the epoch barrier
# (acq_rel add, acquire poll) and sum every slot; the sums must equal the
# sequential simulator's for every round.

@pytest.mark.parametrize("threads,rounds", [(1, 50), (2, 2000), (4, 3000), (7, 500)])
def test_host_threads_match_simulator(threads, rounds):
    out, ns, rc = oracle.host_barrier(threads, rounds, 21)
    assert rc == 0 and ns > 0
    want, _, ctr, rc2 = oracle.slot_rounds(21, rounds, threads, 0)
    assert rc2 == 0 and ctr == rounds * threads
    np.testing.assert_array_equal(out, want)
