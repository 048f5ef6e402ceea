"""GPU parity of the soft epoch barrier workloads against the CPU oracle.

Every comparison is bit-exact (all arithmetic on the path is integer).  Each
test prints the case it is about to launch before the launch.
"""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.fixture(scope="module")
def ccb():
    from cross_core_barrier_amd import ccb as lib
    st, cus, lds, clk = lib.ccb_device_info()
    assert st == 0, lib.ccb_status_string(st)
    return lib


@pytest.fixture(scope="module")
def wl(ccb):
    from cross_core_barrier_amd import workloads
    return workloads


def _u32(t):
    return t.cpu().numpy().view(np.uint32)


# striped / flat / tree x ordering-only / full fences / per-XCD write-back
MODES = [0, 1, 2, 3, 4, 6, 8, 9, 12]
MODE_IDS = ["striped-order", "flat-order", "striped-full", "flat-full", "tree-order", "tree-full",
            "striped-xcd", "flat-xcd", "tree-xcd"]
_oracle_cache = {}


def _oracle_slot(seed, rounds, n_grid, used):
    key = ("slot", seed, rounds, n_grid, used)
    if key not in _oracle_cache:
        _oracle_cache[key] = oracle.slot_rounds(seed, rounds, n_grid, used)
    return _oracle_cache[key]


def _oracle_grouped(seed, rounds, n_grid):
    key = ("grouped", seed, rounds, n_grid)
    if key not in _oracle_cache:
        _oracle_cache[key] = oracle.grouped_rounds(seed, rounds, n_grid)
    return _oracle_cache[key]


# --- witness rounds (whole grid / leading subset) ----------------------------

@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("seed,rounds,n_grid,threads,used,wpc", [
    (0, 100, 8, 64, 0, 0),          # 8 WGs x 64 threads, 100 rounds (small workload)
    (0, 333, 37, 192, 0, 0),        # ragged grid and block, more WGs than stripes
    (7, 257, 37, 128, 19, 0),       # partial participation, odd member count
    (3, 50, 1, 64, 0, 0),           # single participant
    (5, 0, 16, 64, 0, 0),           # zero rounds
    (6, 200, 100, 64, 67, 0),       # stripes with 2 and 3 members
    (8, 91, 300, 64, 0, 0),         # more members than 4 slots per thread
    (9, 2, 5, 64, 0, 0),            # two rounds: the pipeline's prologue and drain only
    (10, 1, 5, 64, 0, 0),           # one round
    (11, 40, 256, 1024, 0, 1),      # 1024-thread workgroups, one per CU
])
def test_slot_rounds_small(wl, seed, rounds, n_grid, threads, used, wpc, mode):
    _say(f"slot_rounds mode={mode} seed={seed} rounds={rounds} grid={n_grid}x{threads} used={used}")
    res = wl.slot_rounds(seed, rounds, n_grid, threads, used, wpc, mode=mode)
    want_out, want_status, want_ctr, rc = _oracle_slot(seed, rounds, n_grid, used)
    assert rc == 0
    assert res.status == 0
    np.testing.assert_array_equal(_u32(res.out), want_out)
    np.testing.assert_array_equal(res.wg_status.cpu().numpy(), want_status)
    assert res.counters == [want_ctr]


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("used", [0, 128])
def test_slot_rounds_grid_full(wl, used, mode):
    """256 WGs x 256 threads, one per CU, 10,000 rounds; then usedCores=128
    with WGs 128..255 idle (the bench's launch configuration)."""
    _say(f"slot_rounds full 256x256 rounds=10000 used={used} wgsPerCu=1 mode={mode}")
    res = wl.slot_rounds(1, 10_000, 256, 256, used, wgs_per_cu=1, mode=mode)
    want_out, want_status, want_ctr, rc = _oracle_slot(1, 10_000, 256, used)
    assert rc == 0 and res.status == 0
    assert res.counters == [want_ctr] == [2_560_000 if used == 0 else 1_280_000]
    np.testing.assert_array_equal(res.wg_status.cpu().numpy(), want_status)
    np.testing.assert_array_equal(_u32(res.out), want_out)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_slot_rounds_largest_coresident_grid(ccb, wl, mode):
    """The largest grid of 64-thread workgroups that the launcher accepts
    (found by bisection: a refused size launches nothing) runs the witness
    rounds bit-exactly, and one workgroup more is refused."""
    n_cu = ccb.ccb_device_info()[1]
    lo, hi = 1, n_cu * 64  # hi: more than any CU holds
    while hi - lo > 1:
        mid = (lo + hi) // 2
        st = wl.slot_rounds(20, 1, mid, 64, check_launch=False, mode=mode).status
        assert st in (ccb.CCB_OK, ccb.CCB_ERR_NOT_CORESIDENT)
        if st == ccb.CCB_OK:
            lo = mid
        else:
            hi = mid
    _say(f"slot_rounds largest grid {lo}x64 rounds=20 mode={mode}")
    assert lo >= n_cu * 8
    res = wl.slot_rounds(20, 20, lo, 64, mode=mode)
    want_out, want_status, want_ctr, rc = _oracle_slot(20, 20, lo, 0)
    assert rc == 0 and res.status == 0
    assert res.counters == [want_ctr] == [20 * lo]
    np.testing.assert_array_equal(res.wg_status.cpu().numpy(), want_status)
    np.testing.assert_array_equal(_u32(res.out), want_out)
    assert wl.slot_rounds(20, 20, lo + 1, 64, check_launch=False, mode=mode).status == \
        ccb.CCB_ERR_NOT_CORESIDENT


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_grouped_largest_coresident_grid(ccb, wl, mode):
    """As above for the grouped rounds (even grids of 64-thread workgroups)."""
    n_cu = ccb.ccb_device_info()[1]
    lo, hi = 1, n_cu * 32  # in pairs of workgroups
    while hi - lo > 1:
        mid = (lo + hi) // 2
        ws = wl.workspace(3)
        slots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * 2 * mid, dtype=torch.int32,
                            device="cuda")
        out = torch.zeros(2 * mid, dtype=torch.int32, device="cuda")
        st = ccb.ccb_run_grouped_rounds(ws, slots, out, None, 4, 1, 2 * mid, 64, 0, 0, mode, None)
        assert st in (ccb.CCB_OK, ccb.CCB_ERR_NOT_CORESIDENT)
        if st == ccb.CCB_OK:
            assert ccb.ccb_syncall_status(ws, 3, None)[0] == ccb.CCB_OK
            lo = mid
        else:
            hi = mid
    n_grid = 2 * lo
    _say(f"grouped largest grid {n_grid}x64 rounds=30 mode={mode}")
    res = wl.grouped_rounds(4, 30, n_grid, 64, mode=mode)
    want_out, want_status, want_ctrs, rc = _oracle_grouped(4, 30, n_grid)
    assert rc == 0 and res.status == 0
    assert tuple(res.counters) == want_ctrs
    np.testing.assert_array_equal(_u32(res.out), want_out)
    ws = wl.workspace(3)
    slots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * (n_grid + 2), dtype=torch.int32,
                        device="cuda")
    out = torch.zeros(n_grid + 2, dtype=torch.int32, device="cuda")
    assert ccb.ccb_run_grouped_rounds(ws, slots, out, None, 4, 1, n_grid + 2, 64, 0, 0, mode,
                                      None) == ccb.CCB_ERR_NOT_CORESIDENT


# --- grouped rounds -----------------------------------------------------------

@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("seed,rounds,n_grid,threads", [(4, 60, 6, 64), (9, 301, 34, 192),
                                                        (2, 150, 130, 64), (3, 77, 300, 64),
                                                        (5, 1, 4, 64), (6, 2, 4, 64),
                                                        (7, 4, 2, 64)])
def test_grouped_small(wl, seed, rounds, n_grid, threads, mode):
    _say(f"grouped mode={mode} seed={seed} rounds={rounds} grid={n_grid}x{threads}")
    res = wl.grouped_rounds(seed, rounds, n_grid, threads, mode=mode)
    want_out, want_status, want_ctrs, rc = _oracle_grouped(seed, rounds, n_grid)
    assert rc == 0 and res.status == 0
    assert tuple(res.counters) == want_ctrs
    np.testing.assert_array_equal(_u32(res.out), want_out)
    np.testing.assert_array_equal(res.wg_status.cpu().numpy(), want_status)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_grouped_full(wl, mode):
    """512 WGs (2 per CU), groups A/B/mix, 100,000 rounds."""
    _say(f"grouped full 512x256 rounds=100000 wgsPerCu=2 mode={mode}")
    res = wl.grouped_rounds(4, 100_000, 512, 256, wgs_per_cu=2, mode=mode)
    want_out, _, want_ctrs, rc = _oracle_grouped(4, 100_000, 512)
    assert rc == 0 and res.status == 0
    assert tuple(res.counters) == want_ctrs == (8_533_504, 8_533_248, 17_066_496)
    np.testing.assert_array_equal(_u32(res.out), want_out)


# --- barrier only ----------------------------------------------------------------

@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_barrier_only_counts_and_placement(wl, mode):
    _say(f"barrier_only 256x256 rounds=1000 wgsPerCu=1 placement mode={mode}")
    st, ctrs, wg, pl = wl.barrier_only(1000, 256, 256, wgs_per_cu=1, placement=True, mode=mode)
    assert st == 0 and ctrs == [256_000]
    assert (wg.cpu().numpy() == 1).all()
    p = pl.cpu().numpy().view(np.uint32).reshape(-1, 2)
    cu = (p[:, 0] >> 8) & 0xF
    sh = (p[:, 0] >> 12) & 0x1
    se = (p[:, 0] >> 13) & 0x7
    key = set(zip(p[:, 1].tolist(), se.tolist(), sh.tolist(), cu.tolist()))
    print(f"distinct CUs used by 256 WGs: {len(key)}; XCDs: {sorted(set(p[:, 1].tolist()))}")
    assert len(set(p[:, 1].tolist())) == 8


@pytest.mark.parametrize("mode", [8, 9, 12], ids=["striped-xcd", "flat-xcd", "tree-xcd"])
@pytest.mark.parametrize("n_grid,used", [(256, 0), (5, 0), (64, 40)])
def test_xcd_registration_and_flags(ccb, wl, n_grid, used, mode):
    """Per-XCD write-back: every member registered once on the XCD it ran on
    (the counts match the placement record), and the flag of each XCD with
    members holds the last round, written by its leader after every round;
    XCDs without members keep count and flag 0."""
    rounds = 300
    members = used or n_grid
    _say(f"barrier_only xcd bookkeeping {n_grid}x64 used={used} rounds={rounds} mode={mode}")
    ws = wl.workspace(1)
    wg = torch.zeros(n_grid, dtype=torch.int32, device="cuda")
    pl = torch.zeros(2 * n_grid, dtype=torch.int32, device="cuda")
    assert ccb.ccb_run_barrier_only(ws, pl, wg, rounds, n_grid, 64, used, 0, 0, mode, None) == 0
    st, ctrs = ccb.ccb_syncall_status(ws, 1, None)
    assert st == 0 and ctrs == [rounds * members]
    xcc = (pl.cpu().numpy().view(np.uint32).reshape(-1, 2)[:members, 1] & 7).astype(np.int64)
    want_counts = np.bincount(xcc, minlength=8)
    w = ws.cpu().numpy()
    counts = w[ccb.CCB_XCD_COUNT_WORD:ccb.CCB_XCD_COUNT_WORD + 8]
    flags = w[ccb.CCB_XCD_FLAG_WORD:ccb.CCB_XCD_FLAG_WORD + 8]
    np.testing.assert_array_equal(counts, want_counts)
    np.testing.assert_array_equal(flags, np.where(want_counts > 0, rounds, 0))


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("n_grid,threads,wpc,rounds", [
    (4096, 64, 16, 200),   # 16 workgroups per CU: 64 members on every stripe
    (256, 1024, 1, 300),   # the largest workgroups, one per CU
])
def test_barrier_only_large_grids(wl, n_grid, threads, wpc, rounds, mode):
    _say(f"barrier_only {n_grid}x{threads} rounds={rounds} wgsPerCu={wpc} mode={mode}")
    st, ctrs, wg, _ = wl.barrier_only(rounds, n_grid, threads, wgs_per_cu=wpc, mode=mode)
    assert st == 0 and ctrs == [rounds * n_grid]
    assert (wg.cpu().numpy() == 1).all()


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_barrier_only_partial(wl, mode):
    _say(f"barrier_only 64x64 rounds=500 used=40 mode={mode}")
    st, ctrs, wg, _ = wl.barrier_only(500, 64, 64, used_cores=40, mode=mode)
    assert st == 0 and ctrs == [500 * 40]
    w = wg.cpu().numpy()
    assert (w[:40] == 1).all() and (w[40:] == 2).all()


# --- failure handling (forced from the host, bounded polls) -------------------------

@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_forced_deadlock_is_reported(ccb, wl, mode):
    """A counter (stripe 0) that starts at 1 (not a multiple of its member
    count) makes the final arrival's target unreachable; the bounded poll
    reports DEADLOCK instead of hanging, and every workgroup exits."""
    _say(f"barrier_only forced deadlock: stripe 0 preset 1, N=4, maxPoll=2000, mode={mode}")
    ws = wl.workspace(1)
    ws[0] = 1
    wg = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = ccb.ccb_run_barrier_only(ws, None, wg, 5, 4, 64, 0, 0, 2000, mode, None)
    assert st == 0
    st, ctrs = ccb.ccb_syncall_status(ws, 1, None)
    assert st == ccb.CCB_ERR_DEADLOCK
    w = wg.cpu().numpy()
    assert (w == 3).any() and set(w.tolist()) <= {1, 3}


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_counter_past_int32_is_invalid_value(ccb, wl, mode):
    """Stripes preset one round below the int32 limit ([SYNCALL] §4.1 types
    the counter int32): the first round still fits and completes, the second
    round's release count would pass INT32_MAX, so every member stores
    INVALID_VALUE in the error word and stops instead of polling for a count
    the counter cannot hold.  Same outcome as the oracle's range-checked
    round simulator on the single counter."""
    n = 4
    flat = (mode & ccb.CCB_BARRIER_FLAT) != 0
    tree = (mode & ccb.CCB_BARRIER_TREE) != 0
    limit = 2**31 - 1
    top = limit // n * n                # last count a round of n can reach

    def preset(ws):
        if flat:
            ws[0] = top - n              # round 1 ends at top, round 2 cannot
        elif tree:
            # 4 groups of one member: the top counter (4 members) fills first
            for g in range(n):
                ws[g * 32] = top // n - 1
            ws[ccb.CCB_TREE_TOP_WORD] = top - n
        else:
            for s in range(n):           # n <= 64 stripes of one member each
                ws[s * 32] = limit - 1

    if flat or tree:
        want_rc1, _ = oracle.epoch_target_checked(top - n, n)
        want_rc2, _ = oracle.epoch_target_checked(top, n)
    else:
        want_rc1, _ = oracle.epoch_target_checked(limit - 1, 1)
        want_rc2, _ = oracle.epoch_target_checked(limit, 1)
    assert (want_rc1, want_rc2) == (oracle.OK, oracle.INVALID_VALUE)
    ws = wl.workspace(1)
    preset(ws)
    _say(f"barrier_only past int32: N={n}, 2 rounds, mode={mode}")
    wg = torch.zeros(n, dtype=torch.int32, device="cuda")
    assert ccb.ccb_run_barrier_only(ws, None, wg, 2, n, 64, 0, 0, 2000, mode, None) == 0
    st, _ = ccb.ccb_syncall_status(ws, 1, None)
    assert st == ccb.CCB_ERR_INVALID_VALUE
    assert (wg.cpu().numpy() == 3).all()
    # one round from the same preset is fine
    ws = wl.workspace(1)
    preset(ws)
    assert ccb.ccb_run_barrier_only(ws, None, wg, 1, n, 64, 0, 0, 2000, mode, None) == 0
    st, ctrs = ccb.ccb_syncall_status(ws, 1, None)
    assert st == ccb.CCB_OK
    if flat:
        assert ctrs == [top]
    elif tree:
        assert ctrs == [top] and int(ws[ccb.CCB_TREE_TOP_WORD]) == top
    else:
        assert ctrs == [n * limit]


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_breakdown_stamps_are_ordered(ccb, wl, mode):
    """ccb_bench_barrier_breakdown: every member's stamps run issue <= reply
    <= release within a round and release <= next issue across rounds; no
    member is released before the round's last arrival was issued; every
    arrival is counted."""
    n, rounds = 64, 200
    _say(f"barrier breakdown: {n} x 256, {rounds} rounds, mode={mode}")
    ws = wl.workspace(1)
    stamps = torch.zeros(rounds * n * 3, dtype=torch.int64, device="cuda")
    assert ccb.ccb_bench_barrier_breakdown(ws, stamps, rounds, n, 256, 0, mode, None) == 0
    st, ctrs = ccb.ccb_syncall_status(ws, 1, None)
    assert st == 0 and ctrs == [rounds * n]
    t = stamps.cpu().numpy().reshape(rounds, n, 3)
    assert (t > 0).all()
    assert (t[:, :, 0] <= t[:, :, 1]).all() and (t[:, :, 1] <= t[:, :, 2]).all()
    assert (t[1:, :, 0] >= t[:-1, :, 2]).all()
    # the barrier: a release in round r follows every round-r arrival's issue
    assert (t[:, :, 2].min(axis=1) >= t[:, :, 0].max(axis=1)).all()


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_grouped_timeline_matches_oracle(ccb, wl, mode):
    """ccb_bench_grouped_timeline computes what ccb_run_grouped_rounds does
    (the oracle's outputs) and stamps each member's own rounds in order:
    an even member's rounds are A and mix, an odd member's B and mix."""
    n, rounds = 16, 60
    _say(f"grouped timeline: {n} x 64, {rounds} rounds, mode={mode}")
    ws = wl.workspace(3)
    slots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * n, dtype=torch.int32, device="cuda")
    out = torch.zeros((rounds, n), dtype=torch.int32, device="cuda")
    stamps = torch.zeros(rounds * n, dtype=torch.int64, device="cuda")
    assert ccb.ccb_bench_grouped_timeline(ws, slots, out, stamps, 4, rounds, n, 64, 0, mode) == 0
    st, ctrs = ccb.ccb_syncall_status(ws, 3, None)
    want_out, _, want_ctrs, rc = oracle.grouped_rounds(4, rounds, n)
    assert st == 0 and rc == 0 and tuple(ctrs) == want_ctrs
    assert np.array_equal(_u32(out), want_out)
    t = stamps.cpu().numpy().reshape(rounds, n)
    own = rounds // 3 * 2   # rounds divisible by 3: each member takes 2 of every 3
    assert (t[:own] > 0).all() and (t[own:] == 0).all()
    assert (np.diff(t[:own], axis=0) >= 0).all()


def test_breakdown_rejects_bad_arguments(ccb, wl):
    ws = wl.workspace(1)
    stamps = torch.zeros(8 * 3, dtype=torch.int64, device="cuda")
    assert ccb.ccb_bench_barrier_breakdown(ws, None, 1, 8, 64) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_bench_barrier_breakdown(ws, stamps, 0, 8, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_barrier_breakdown(ws, stamps, ccb.CCB_BREAKDOWN_MAX_ROUNDS + 1, 8,
                                           64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_barrier_breakdown(ws, stamps.data_ptr() + 4, 1, 8, 64) == \
        ccb.CCB_ERR_INVALID_VALUE


def test_reset_clears_error_word(ccb, wl):
    ws = wl.workspace(1)
    ws[0] = 5
    ws[32] = 3
    ws[ccb.CCB_STRIPES * 32] = ccb.CCB_ERR_DEADLOCK
    assert ccb.ccb_syncall_workspace_reset(ws, 1, None) == 0
    torch.cuda.synchronize()
    assert int(ws.abs().sum()) == 0
    assert ccb.ccb_syncall_status(ws, 1, None) == (0, [0])


def test_status_sums_stripes_of_many_barriers(ccb, wl):
    """ccb_syncall_status reads each stripe's counter word (not the rest of its
    line) over 130 barriers, more than one host chunk of 64, and sums the 64
    stripes of each barrier in int64: barrier 77's stripes hold 2^30 - 1
    each, a total past 2^31."""
    nb = 130
    _say(f"syncall_status over {nb} barriers")
    ws = wl.workspace(nb)
    lines = ws.view(-1, 32)
    b = torch.arange(nb, device="cuda", dtype=torch.int32).repeat_interleave(ccb.CCB_STRIPES)
    k = torch.arange(ccb.CCB_STRIPES, device="cuda", dtype=torch.int32).repeat(nb)
    lines[: nb * ccb.CCB_STRIPES, 0] = b * 1000 + k
    lines[: nb * ccb.CCB_STRIPES, 1:] = -7  # rest of each line: not counted
    lines[77 * ccb.CCB_STRIPES: 78 * ccb.CCB_STRIPES, 0] = 2**30 - 1
    st, arr = ccb.ccb_syncall_status(ws, nb, None)
    assert st == ccb.CCB_OK
    want = [bb * 1000 * 64 + 63 * 64 // 2 for bb in range(nb)]
    want[77] = 64 * (2**30 - 1)
    assert arr == want
    lines[nb * ccb.CCB_STRIPES, 0] = ccb.CCB_ERR_DEADLOCK
    st, arr2 = ccb.ccb_syncall_status(ws, nb, None)
    assert st == ccb.CCB_ERR_DEADLOCK and arr2 == want


@pytest.mark.parametrize("raw", [False, True], ids=["torch-stream", "raw-handle"])
def test_helpers_on_a_side_stream(ccb, wl, raw):
    """The torch-side helpers order their launches on a caller's stream after
    their own fills, and the caller's current stream after the launch."""
    _say(f"helpers on a side stream (raw handle: {raw})")
    s = torch.cuda.Stream()
    arg = s.cuda_stream if raw else s
    res = wl.slot_rounds(0, 100, 8, 64, stream=arg)
    want_out, _, want_ctr, rc = _oracle_slot(0, 100, 8, 0)
    assert rc == 0 and res.status == 0 and res.counters == [want_ctr]
    assert np.array_equal(_u32(res.out), want_out)
    from cross_core_barrier_amd import inputs
    x = inputs.stencil_input(2, 70_001)
    st, y = wl.stencil(torch.from_numpy(x).cuda(), 5, 16, 128, stream=arg)
    assert st == 0 and np.array_equal(y.cpu().numpy(), oracle.stencil(x, 5))
    val, meta, rows = inputs.cnt_batch_input(3, 4100, 16, small_values=True)
    err, final, rel = wl.cnt_batch(torch.from_numpy(val.view(np.int32)).cuda(),
                                   torch.from_numpy(meta).cuda(), rows, stream=arg)
    want_final, want_rel, rc = oracle.cnt_batch(val, meta, rows)
    assert rc == 0 and int(err.item()) == 0
    assert np.array_equal(final.cpu().numpy().view(np.uint32), want_final)
    assert np.array_equal(rel.cpu().numpy(), want_rel)


def test_concurrent_launches_from_host_threads(ccb, wl):
    """Four host threads, each with its own stream and workspace, launch
    barrier-only grids over and over with different wgsPerCu (so each sets
    the kernel's dynamic-LDS limit differently) and barrier variants.  Every
    launch is accepted and every count is exact.  The grids are small enough
    (16 workgroups) that all four fit on the device together."""
    import threading
    _say("barrier_only from 4 host threads x 20 launches, 16 WGs each")
    n, rounds, reps = 16, 500, 20
    wss = [wl.workspace(1) for _ in range(4)]
    streams = [torch.cuda.Stream() for _ in range(4)]
    torch.cuda.synchronize()
    results = [[] for _ in range(4)]

    def worker(t):
        for i in range(reps):
            mode = MODES[(t + i) % len(MODES)]
            st = ccb.ccb_syncall_workspace_reset(wss[t], 1, streams[t])
            if st == 0:
                st = ccb.ccb_run_barrier_only(wss[t], None, None, rounds, n, 64, 0, 1 + t, 0,
                                              mode, streams[t])
            got = ccb.ccb_syncall_status(wss[t], 1, streams[t]) if st == 0 else (st, None)
            results[t].append((st, got))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads)
    for t in range(4):
        assert len(results[t]) == reps
        for st, got in results[t]:
            assert st == 0 and got == (0, [rounds * n]), (t, st, got)


def test_not_coresident_rejected(ccb, wl):
    _say("barrier_only oversize grid: expect NOT_CORESIDENT, nothing launched")
    ws = wl.workspace(1)
    st = ccb.ccb_run_barrier_only(ws, None, None, 1, 256 * 64, 1024, 0, 0, 100, 0, None)
    assert st == ccb.CCB_ERR_NOT_CORESIDENT
    assert ccb.ccb_syncall_status(ws, 1, None) == (0, [0])


def test_invalid_arguments(ccb, wl):
    ws = wl.workspace(1)
    assert ccb.ccb_run_barrier_only(ws, None, None, 1, 8, 65) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_barrier_only(ws, None, None, 1, 8, 64, 9) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_barrier_only(ws, None, None, 1, 8, 64, -1) == ccb.CCB_ERR_INVALID_VALUE
    for bad in (5, 7, 10, 13, 14, 16, -1):
        assert ccb.ccb_run_barrier_only(ws, None, None, 1, 8, 64, mode=bad) == \
            ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_barrier_only(ws.data_ptr() + 4, None, None, 1, 8, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_grouped_rounds(ws, ws, ws, None, 0, 1, 7, 64) == ccb.CCB_ERR_INVALID_VALUE
