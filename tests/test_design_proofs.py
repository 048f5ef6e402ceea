"""Brute-force proofs of the kernels' barrier designs (CPU).

The kernels split each counter into stripes (or, as the tree variant, into
group counters under a top counter), the ordering-only witness kernels
pipeline their rounds two deep, and full visibility can be placed as one L2
write-back per XCD.  None of that is in the pages; each must compute
exactly what the pages' single-counter barrier computes.  The model
is tests/design_models.py, built on the oracle's round specifications; the
first test checks that with one stripe and the plain program it explores
exactly the oracle's own state space.
"""

import pytest

from oracle import enumerate as en

import design_models as dm


@pytest.mark.parametrize("p,r", [(2, 3), (3, 3), (3, 2)])
def test_single_stripe_is_the_oracles_barrier(p, r):
    ref = en.enumerate_schedules(en.whole_grid(p, r), p)
    got = dm.explore(en.whole_grid(p, r), p, layout=dm.Striped(1))
    assert (got.deadlock, got.violations, got.final_counters) == \
        (ref.deadlock, ref.violations, ref.final_counters)
    assert got.states == ref.states
    for kw in ({"poll_cmp": "eq"}, {"skip": [(1, 0)]}, {"counter_init": [1]}):
        ref = en.enumerate_schedules(en.whole_grid(p, r), p, **kw)
        got = dm.explore(en.whole_grid(p, r), p, layout=dm.Striped(1), **kw)
        assert (got.deadlock, len(got.violations) > 0) == (ref.deadlock, len(ref.violations) > 0)


# --- striped counters ------------------------------------------------------------

@pytest.mark.parametrize("p,r,k", [(2, 3, 2), (3, 3, 2), (3, 2, 3), (3, 3, 4)])
def test_striped_whole_grid(p, r, k):
    res = dm.explore(en.whole_grid(p, r), p, layout=dm.Striped(k))
    assert not res.deadlock and res.violations == []
    assert res.final_counters == {(r * p,)}


def test_striped_partial_and_oversized_n():
    res = dm.explore(en.whole_grid(3, 3, used_cores=2, n_members=2), 3, layout=dm.Striped(2))
    assert not res.deadlock and res.violations == [] and res.final_counters == {(6,)}
    res = dm.explore(en.whole_grid(2, 1, used_cores=3, n_members=2), 2, layout=dm.Striped(2))
    assert res.deadlock


def test_striped_negative_controls():
    assert dm.explore(en.whole_grid(2, 2), 2, layout=dm.Striped(2), poll_cmp="eq").deadlock
    assert dm.explore(en.whole_grid(3, 2), 3, layout=dm.Striped(2), skip=[(1, 0)]).deadlock
    res = dm.explore(en.whole_grid(3, 3), 3, layout=dm.Striped(2), counter_init=[1])
    assert res.violations != [] or res.deadlock


# --- two-level tree ----------------------------------------------------------------

@pytest.mark.parametrize("p,r,g", [(2, 3, 2), (3, 3, 2), (4, 2, 2), (3, 3, 3), (4, 2, 3),
                                   (3, 2, 4)])
def test_tree_whole_grid(p, r, g):
    res = dm.explore(en.whole_grid(p, r), p, layout=dm.Tree(g))
    assert not res.deadlock and res.violations == []
    assert res.final_counters == {(r * p,)}


def test_tree_partial_grouped_and_pipelined():
    res = dm.explore(en.whole_grid(4, 2, used_cores=3, n_members=3), 4, layout=dm.Tree(2))
    assert not res.deadlock and res.violations == [] and res.final_counters == {(6,)}
    g = en.grouped(4, 6)
    res = dm.explore(g, 4, layout=dm.Tree(2), ring_depth=4)
    assert not res.deadlock and res.violations == [] and res.final_counters == {(4, 4, 8)}
    res = dm.explore(en.whole_grid(3, 4), 3, layout=dm.Tree(2), write_lead=2, read_lag=2,
                     ring_depth=4)
    assert not res.deadlock and res.violations == [] and res.final_counters == {(12,)}


def test_tree_negative_controls():
    assert dm.explore(en.whole_grid(2, 2), 2, layout=dm.Tree(2), poll_cmp="eq").deadlock
    assert dm.explore(en.whole_grid(3, 2), 3, layout=dm.Tree(2), skip=[(1, 0)]).deadlock
    res = dm.explore(en.whole_grid(3, 3), 3, layout=dm.Tree(2), counter_init=[1])
    assert res.violations != [] or res.deadlock
    res = dm.explore(en.whole_grid(2, 1, used_cores=3, n_members=2), 2, layout=dm.Tree(2))
    assert res.deadlock


# --- the pipelined (early-write) schedules ---------------------------------------
# With ordering-only visibility the witness kernels write the next round's
# witness right after passing a barrier.

@pytest.mark.parametrize("k", [1, 2])
def test_early_write_ring_depths(k):
    # whole grid: a writer can lead a reader by one round -> 2 rows suffice
    kw = {"layout": dm.Striped(k), "write_lead": 1, "read_lag": 1}
    assert dm.explore(en.whole_grid(3, 3), 3, ring_depth=2, **kw).violations == []
    assert dm.explore(en.whole_grid(3, 3), 3, ring_depth=1, **kw).violations != []
    # grouped A/B/mix: 4 rows are needed and suffice
    g = en.grouped(4, 6)
    res4 = dm.explore(g, 4, ring_depth=4, **kw)
    assert not res4.deadlock and res4.violations == [] and res4.final_counters == {(4, 4, 8)}
    assert dm.explore(g, 4, ring_depth=3, **kw).violations != []


def test_early_write_grouped_longer():
    res = dm.explore(en.grouped(4, 9), 4, layout=dm.Striped(2), write_lead=1, read_lag=1,
                     ring_depth=4)
    assert not res.deadlock and res.violations == [] and res.final_counters == {(6, 6, 12)}


# The two-deep pipeline of the ordered witness kernels: a member writes the
# witness of its own round i + 2 right after passing round i's barrier, and
# may still be reading round i's row until it arrives at round i + 2.  A ring
# of D rows is safe exactly when the writer cannot reach a row again while a
# reader is still on it; the brute force fixes the smallest D for each
# pattern (the kernels use six rows for both).

@pytest.mark.parametrize("k", [1, 2])
def test_two_deep_pipeline_whole_grid(k):
    kw = {"layout": dm.Striped(k), "write_lead": 2, "read_lag": 2}
    for p, r in ((3, 4), (4, 6)):
        res = dm.explore(en.whole_grid(p, r), p, ring_depth=4, **kw)
        assert not res.deadlock and res.violations == [] and res.final_counters == {(p * r,)}
        assert dm.explore(en.whole_grid(p, r), p, ring_depth=3, **kw).violations != []
    res = dm.explore(en.whole_grid(3, 4, used_cores=2, n_members=2), 3, ring_depth=4, **kw)
    assert not res.deadlock and res.violations == [] and res.final_counters == {(8,)}


@pytest.mark.parametrize("k", [1, 2])
def test_two_deep_pipeline_grouped(k):
    kw = {"layout": dm.Striped(k), "write_lead": 2, "read_lag": 2}
    for p, r in ((4, 9), (4, 12), (5, 9)):
        g = en.grouped(p, r)
        res = dm.explore(g, p, ring_depth=6, **kw)
        assert not res.deadlock and res.violations == []
        assert res.final_counters == {en.expected_final_counters(g)}
    assert dm.explore(en.grouped(4, 12), 4, ring_depth=5, **kw).violations != []


def test_lead_plus_lag_bound():
    # whole grid: safe exactly when write lead + read lag <= D
    for a in (1, 2, 3):
        for b in (1, 2, 3):
            for d in (a + b - 1, a + b):
                # enough rounds for the writer to come back to the same row
                res = dm.explore(en.whole_grid(3, d + 2), 3, write_lead=a, read_lag=b,
                                 ring_depth=d)
                assert (res.violations == []) == (d >= a + b), (a, b, d)


# --- full visibility with one L2 write-back per XCD ----------------------------------

@pytest.mark.parametrize("p,r,xcd_of,k", [(3, 3, (0, 1, 0), 1), (3, 3, (0, 1, 0), 2),
                                          (4, 2, (0, 1, 0, 1), 2), (3, 2, (0, 0, 0), 1),
                                          (4, 2, (0, 1, 2, 0), 1)])
def test_xcd_writeback_whole_grid(p, r, xcd_of, k):
    """Writes sit in the writer's XCD L2 until its leader writes back; every
    read after the flag poll still sees every member's write of the round."""
    res = dm.explore_xcd(en.whole_grid(p, r), p, xcd_of, k=k)
    assert not res.deadlock and res.violations == []
    assert res.final_counters == {(r * p,)}


def test_xcd_writeback_grouped_and_partial():
    res = dm.explore_xcd(en.grouped(4, 6), 4, (0, 1, 1, 0), ring_depth=4)
    assert not res.deadlock and res.violations == [] and res.final_counters == {(4, 4, 8)}
    res = dm.explore_xcd(en.whole_grid(4, 3, used_cores=3, n_members=3), 4, (0, 1, 1, 0), k=2)
    assert not res.deadlock and res.violations == [] and res.final_counters == {(9,)}


@pytest.mark.parametrize("variant", ["early_writeback", "no_writeback", "no_flag_poll",
                                     "own_flag_only"])
def test_xcd_writeback_negative_controls(variant):
    """Each shortcut lets some read see a stale value."""
    res = dm.explore_xcd(en.whole_grid(3, 3), 3, (0, 1, 0), variant=variant)
    assert res.violations != []


def test_xcd_writeback_shallow_ring():
    assert dm.explore_xcd(en.whole_grid(3, 3), 3, (0, 1, 0), ring_depth=1).violations != []
