"""ccb_run_stencil_noalloc: the allocation-free stencil entry point against
the existing one (ccb_run_stencil with caller scratch), bit for bit, on two
calls in a row with the second one smaller, in every barrier variant; plus
the oracle on the smaller case and the scratch-size limit.

Each test prints the case it is about to launch before the launch.
"""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# striped / flat / tree x ordering-only / full fences / per-XCD write-back
MODES = [0, 1, 2, 3, 4, 6, 8, 9, 12]
MODE_IDS = ["striped-order", "flat-order", "striped-full", "flat-full", "tree-order", "tree-full",
            "striped-xcd", "flat-xcd", "tree-xcd"]


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.fixture(scope="module")
def ccb():
    from cross_core_barrier_amd import ccb as lib
    st, _, _, _ = lib.ccb_device_info()
    assert st == 0, lib.ccb_status_string(st)
    return lib


@pytest.fixture(scope="module")
def wl(ccb):
    from cross_core_barrier_amd import workloads
    return workloads


def _noalloc(ccb, x, iters, n_grid, threads, mode, stream=None):
    a = x.clone()
    b = torch.empty_like(a)
    status = torch.full((1,), -1, dtype=torch.int32, device=x.device)
    torch.cuda.synchronize()
    st = ccb.ccb_run_stencil_noalloc(a, b, a.numel(), iters, status, n_grid, threads, 0, 0, mode,
                                     stream)
    assert st == ccb.CCB_OK, ccb.ccb_status_string(st)
    torch.cuda.synchronize()
    return int(status.item()), (a if iters % 2 == 0 else b)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_noalloc_matches_scratch_entry_point_twice(ccb, wl, mode):
    from cross_core_barrier_amd import inputs
    cases = [(1_000_003, 7, 64, 256), (50_001, 5, 16, 128)]  # the second call is smaller
    for n, iters, n_grid, threads in cases:
        x = torch.from_numpy(inputs.stencil_input(2, n)).cuda()
        _say(f"stencil_noalloc n={n} iters={iters} grid={n_grid}x{threads} mode={mode}")
        st_out, y = _noalloc(ccb, x, iters, n_grid, threads, mode)
        assert st_out == ccb.CCB_OK
        _say(f"stencil (caller scratch) n={n} iters={iters} grid={n_grid}x{threads} mode={mode}")
        st, want = wl.stencil(x, iters, n_grid, threads, mode=mode)
        assert st == ccb.CCB_OK
        assert torch.equal(y, want)
    # the smaller case also against the oracle
    x_np = inputs.stencil_input(2, cases[-1][0])
    assert np.array_equal(y.cpu().numpy(), oracle.stencil(x_np, cases[-1][1]))


def test_noalloc_on_a_side_stream_and_full_size(ccb, wl):
    """The benchmark's shape (2^26 elements, 1024 x 256, 8 iterations here)
    on a non-default stream, against the caller-scratch entry point."""
    from cross_core_barrier_amd import inputs
    n, iters = 1 << 26, 8
    x = torch.from_numpy(inputs.stencil_input(2, n)).cuda()
    s = torch.cuda.Stream()
    _say(f"stencil_noalloc n=2^26 iters={iters} grid=1024x256 on a side stream")
    st_out, y = _noalloc(ccb, x, iters, 1024, 256, 0, s)
    assert st_out == ccb.CCB_OK
    _say(f"stencil (caller scratch) n=2^26 iters={iters} grid=1024x256")
    st, want = wl.stencil(x, iters, 1024, 256, wgs_per_cu=4)
    assert st == ccb.CCB_OK
    assert torch.equal(y, want)


def test_noalloc_reports_deadlock_through_status(ccb):
    """A grid one workgroup larger than the members that can call would hang a
    barrier; it cannot be made here, so the deadlock path is driven by a poll
    bound of 1 on a multi-workgroup launch instead: if any member gives up,
    *statusOut carries CCB_ERR_DEADLOCK, and the next call starts from a
    cleared workspace again (its status is CCB_OK)."""
    from cross_core_barrier_amd import inputs
    x = torch.from_numpy(inputs.stencil_input(2, 200_000)).cuda()
    a, b = x.clone(), torch.empty_like(x)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    _say("stencil_noalloc with maxPoll=1 on 64 workgroups")
    st = ccb.ccb_run_stencil_noalloc(a, b, a.numel(), 40, status, 64, 256, 0, 1, 0, None)
    assert st == ccb.CCB_OK
    torch.cuda.synchronize()
    assert int(status.item()) in (ccb.CCB_OK, ccb.CCB_ERR_DEADLOCK)
    _say("stencil_noalloc again with the default poll bound")
    st_out, y = _noalloc(ccb, x, 3, 64, 256, 0)
    assert st_out == ccb.CCB_OK
    assert np.array_equal(y.cpu().numpy(), oracle.stencil(x.cpu().numpy(), 3))


def test_noalloc_rejects_launches_beyond_its_scratch(ccb):
    # ordering-only: halo of 2 x 1024 x 257 chunks x 2 int32 = 4.2 MB > 4 MiB
    n = (1 << 28) + (1 << 20)
    a = 1 << 44
    b = a + n * 4 + 4096
    assert ccb.ccb_stencil_halo_bytes(n, 256, 1024) + 8448 > ccb.CCB_NOALLOC_SCRATCH_BYTES
    assert ccb.ccb_run_stencil_noalloc(a, b, n, 2, None, 1024, 256, 0, 0, 0) == \
        ccb.CCB_ERR_INVALID_VALUE
    status = torch.zeros(2, dtype=torch.int32, device="cuda")
    x = torch.zeros(1024, dtype=torch.int32, device="cuda")
    y = torch.zeros(1024, dtype=torch.int32, device="cuda")
    assert ccb.ccb_run_stencil_noalloc(x, y, 1024, 2, status.data_ptr() + 2, 4, 64) == \
        ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_stencil_noalloc(None, y, 1024, 2, status, 4, 64) == \
        ccb.CCB_ERR_NULL_POINTER
