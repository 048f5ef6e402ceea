"""GPU checks of the floor microbenchmarks and of HIP's grid barrier as the
library launches them: each one's observable result (the final count of an
atomic chain, a copy bit for bit, the completion word of the grid sync), and
that a launch the runtime refuses leaves no error behind for the caller."""

import numpy as np
import pytest

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


@pytest.mark.parametrize("kind", [0, 1], ids=["fetch-add", "load"])
@pytest.mark.parametrize("fenced", [0, 1], ids=["plain", "fenced"])
def test_atomic_chain(ccb, kind, fenced):
    _say(f"atomic chain kind={kind} fenced={fenced} iters=1000")
    line = torch.zeros(64, dtype=torch.int32, device="cuda")
    ticks = torch.zeros(2, dtype=torch.int64, device="cuda")
    ccb.check(ccb.ccb_bench_atomic_chain(line, ticks, 1000, fenced, kind), "chain")
    torch.cuda.synchronize()
    # a fetch-add chain adds one per step; a load chain leaves the line alone
    assert int(line[0].item()) == (1000 if kind == 0 else 0)
    assert int(line[1:].abs().sum().item()) == 0
    t = ticks.cpu().numpy()
    assert t[1] > t[0] > 0


def test_atomic_contended(ccb):
    n_grid, iters = 256, 200
    _say(f"contended fetch-add {n_grid} workgroups x {iters}")
    line = torch.zeros(64, dtype=torch.int32, device="cuda")
    ticks = torch.zeros(2 * n_grid, dtype=torch.int64, device="cuda")
    ccb.check(ccb.ccb_bench_atomic_contended(line, ticks, iters, n_grid), "contended")
    torch.cuda.synchronize()
    assert int(line[0].item()) == n_grid * iters
    t = ticks.cpu().numpy().reshape(n_grid, 2)
    assert np.all(t[:, 1] > t[:, 0])


@pytest.mark.parametrize("peer", [1, 8, 255])
def test_notify_pingpong(ccb, peer):
    iters = 2000
    _say(f"notify ping-pong workgroups 0 and {peer}, {iters} turns")
    lines = torch.zeros(64, dtype=torch.int32, device="cuda")
    ticks = torch.zeros(4, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ccb.check(ccb.ccb_bench_notify_pingpong(lines, ticks, iters, peer, 0, err), "ping-pong")
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert int(lines[0].item()) == iters and int(lines[32].item()) == iters
    assert int(lines[1:32].abs().sum().item()) == 0 and int(lines[33:].abs().sum().item()) == 0
    t = ticks.cpu().numpy()
    assert t[1] > t[0] > 0
    assert 0 <= t[2] < 8 and 0 <= t[3] < 8  # XCC ids


def test_notify_pingpong_forced_deadlock(ccb):
    """Line B preset to -5: after the partner's first turn it holds -4, so
    workgroup 0 never sees turn 1 and the partner never sees turn 2.  Both
    waits run out after maxPoll polls and report DEADLOCK; nothing hangs."""
    _say("notify ping-pong forced deadlock, maxPoll=2000")
    lines = torch.zeros(64, dtype=torch.int32, device="cuda")
    lines[32] = -5
    ticks = torch.zeros(4, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ccb.check(ccb.ccb_bench_notify_pingpong(lines, ticks, 10, 1, 2000, err), "ping-pong")
    torch.cuda.synchronize()
    assert int(err.item()) == ccb.CCB_ERR_DEADLOCK
    assert int(lines[0].item()) == 1 and int(lines[32].item()) == -4


@pytest.mark.parametrize("n_words", [4, 4 * 1000003, 1 << 24])
def test_copy_bit_exact(ccb, n_words):
    _say(f"copy {n_words * 4} bytes")
    g = torch.Generator(device="cuda")
    g.manual_seed(n_words)
    src = torch.randint(-2**31, 2**31 - 1, (n_words + 4,), dtype=torch.int32, device="cuda",
                        generator=g)
    dst = torch.full_like(src, 7)
    ccb.check(ccb.ccb_bench_copy(dst, src, n_words * 4), "copy")
    torch.cuda.synchronize()
    assert torch.equal(dst[:n_words], src[:n_words])
    assert torch.all(dst[n_words:] == 7)  # nothing past nBytes


def test_copy_zero_bytes(ccb):
    src = torch.ones(4, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    ccb.check(ccb.ccb_bench_copy(dst, src, 0), "copy 0")
    torch.cuda.synchronize()
    assert int(dst.sum().item()) == 0


@pytest.mark.parametrize("n_grid,threads,rounds", [(2, 64, 10), (256, 256, 50), (1024, 256, 20)])
def test_hip_grid_sync_completes(ccb, n_grid, threads, rounds):
    _say(f"HIP grid sync {n_grid} x {threads}, {rounds} rounds")
    done = torch.zeros(1, dtype=torch.int32, device="cuda")
    ccb.check(ccb.ccb_bench_hip_grid_sync(rounds, n_grid, threads, done), "grid sync")
    torch.cuda.synchronize()
    assert int(done.item()) == rounds


def test_oversized_grid_sync_refused(ccb):
    _say("HIP grid sync refused on the host: 16384 x 1024")
    done = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert ccb.ccb_bench_hip_grid_sync(1, 16384, 1024, done) == ccb.CCB_ERR_NOT_CORESIDENT
    torch.cuda.synchronize()
    assert int(done.item()) == 0


def test_refused_launch_leaves_no_error(ccb):
    """The runtime refuses a cooperative grid larger than can be resident
    (65536 one-wave workgroups; at most 32 fit a CU).  The status says so, and
    the caller's next launches, torch's and the library's, run normally.  The
    kernel's workgroups never wait on each other and the tick buffer covers
    every workgroup, so the request is safe even if it were launched."""
    n_grid = 65536
    _say(f"contended fetch-add refused by the runtime: {n_grid} workgroups")
    line = torch.zeros(64, dtype=torch.int32, device="cuda")
    ticks = torch.zeros(2 * n_grid, dtype=torch.int64, device="cuda")
    assert ccb.ccb_bench_atomic_contended(line, ticks, 1, n_grid) == ccb.CCB_ERR_NOT_CORESIDENT
    x = torch.arange(8, device="cuda", dtype=torch.int32) * 3  # raises if an error was left
    torch.cuda.synchronize()
    assert int(x.sum().item()) == 84
    done = torch.zeros(1, dtype=torch.int32, device="cuda")
    ccb.check(ccb.ccb_bench_hip_grid_sync(3, 8, 64, done), "grid sync after refusal")
    torch.cuda.synchronize()
    assert int(done.item()) == 3


@pytest.mark.parametrize("variant", range(6))
def test_fence_placement_completes(ccb, variant):
    """Every placement runs its rounds without a bounded wait giving up; the
    two that release and acquire at agent scope for every reader (every
    workgroup, or one write-back per XCD plus every workgroup's acquire)
    never return a stale value to a plain read after the barrier."""
    n, rounds = 64, 300
    _say(f"fence placement variant {variant}: {n} x 64, {rounds} rounds")
    nbytes = ccb.ccb_bench_fence_placement_bytes(n)
    scratch = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    stale = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    assert ccb.ccb_bench_fence_placement(scratch, nbytes, stale, rounds, n, 64, variant) == 0
    torch.cuda.synchronize()
    assert int(scratch[ccb.CCB_STRIPES * 32].item()) == 0          # error word
    s = stale.cpu().numpy()
    assert ((s >= 0) & (s <= rounds)).all()
    if variant in (1, 4):
        assert (s == 0).all()
    assert ccb.ccb_bench_fence_placement(scratch, nbytes - 4, stale, rounds, n, 64, variant) == \
        ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_fence_placement(scratch, nbytes, stale, rounds, n, 64, 6) == \
        ccb.CCB_ERR_INVALID_VALUE
