"""GPU parity of the in-kernel barrier API (include/ccb_device.h) used as a
caller's own kernel would use it: ccb_syncall_soft / _ordered / _flat /
_bounded / _mix and the split-phase ccb_arrive / ccb_await inside the flag-slot pattern of the SYNCALL guide §6.1, on 2-D
grids, with and without a usedCores subset.  The test kernels live in
tests/devapi (built by __graft_entry__.build()); the expected sums come from
the oracle's witness rounds."""

import ctypes
import os

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LIB = os.path.join(os.path.dirname(__file__), "devapi", "libccb_devapi.so")
VARIANTS = {0: "soft", 1: "soft_ordered", 2: "soft_flat", 3: "soft_bounded",
            6: "split_phase", 7: "soft_tree", 8: "soft_xcd"}  # 4, 5: mix 1:1, 1:2


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.fixture(scope="module")
def devapi():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB)
    V, I32, U32, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64
    lib.devapi_run.restype = ctypes.c_int
    lib.devapi_run.argtypes = [ctypes.c_int, V, V, V, V, U64, I32, I32, I32, I32, I32, U32, V]
    return lib


def _run(lib, variant, gx, gy, threads, used, rounds, seed, max_poll=0, preset=None):
    from cross_core_barrier_amd import ccb, workloads
    n_grid = gx * gy
    ws = workloads.workspace(1)
    if preset is not None:
        ws[0] = preset
    slots = torch.zeros(2 * n_grid, dtype=torch.int32, device="cuda")
    out = torch.zeros(max(rounds, 1) * n_grid, dtype=torch.int32, device="cuda")
    status = torch.zeros(n_grid, dtype=torch.int32, device="cuda")
    rc = lib.devapi_run(variant, ws.data_ptr(), slots.data_ptr(), out.data_ptr(), status.data_ptr(),
                        seed, rounds, gx, gy, threads, used, max_poll, None)
    assert rc == 0, rc
    torch.cuda.synchronize()
    st, ctrs = ccb.ccb_syncall_status(ws, 1, None)
    return st, ctrs, out.cpu().numpy().view(np.uint32).reshape(-1, n_grid)[:rounds], status.cpu().numpy()


@pytest.mark.parametrize("variant", list(VARIANTS), ids=list(VARIANTS.values()))
@pytest.mark.parametrize("gx,gy,threads,used,rounds,seed", [
    (8, 4, 64, 0, 60, 11),       # 2-D grid, whole grid
    (5, 3, 128, 7, 41, 12),      # leading subset of a 2-D grid, idle workgroups
    (16, 16, 256, 0, 30, 13),    # 256 workgroups, more than the stripes
    (3, 1, 1024, 0, 25, 14),     # 1024-thread workgroups
    (1, 1, 64, 0, 10, 15),       # a single participant
])
def test_device_api_witness_rounds(devapi, variant, gx, gy, threads, used, rounds, seed):
    _say(f"device api {VARIANTS[variant]} grid={gx}x{gy}x{threads} used={used} rounds={rounds}")
    st, ctrs, out, status = _run(devapi, variant, gx, gy, threads, used, rounds, seed,
                                 max_poll=1_000_000)
    n_grid = gx * gy
    members = used if used else n_grid
    want_out, want_status, want_ctr, rc = oracle.slot_rounds(seed, rounds, n_grid, used)
    assert rc == 0 and st == 0
    assert ctrs == [want_ctr] == [rounds * members]
    np.testing.assert_array_equal(out[:, :members], want_out[:, :members])
    np.testing.assert_array_equal(status, want_status)


@pytest.mark.parametrize("variant,ratio", [(4, 1), (5, 2)], ids=["mix_1_1", "mix_1_2"])
@pytest.mark.parametrize("gx,gy,groups,rounds,seed", [
    (8, 2, 5, 40, 16),     # 5 groups, idle workgroups after them
    (12, 1, 0, 33, 17),    # groups == 0: the whole grid
    (9, 3, 4, 20, 18),
])
def test_device_api_mixed_roles(devapi, variant, ratio, gx, gy, groups, rounds, seed):
    """Role groups (one leader and `ratio` companions, [SYNCALL] §4.2's
    groups x (1 + ratio) participants): the sums over the participants match
    the oracle's witness rounds with that many members."""
    n_grid = gx * gy
    members = oracle.mix_participants(groups, ratio, n_grid)
    _say(f"device api soft_mix 1:{ratio} grid={gx}x{gy} groups={groups} members={members}")
    st, ctrs, out, status = _run(devapi, variant, gx, gy, 64, groups, rounds, seed)
    want_out, want_status, want_ctr, rc = oracle.slot_rounds(seed, rounds, n_grid,
                                                             members if groups else 0)
    assert rc == 0 and st == 0
    assert ctrs == [want_ctr] == [rounds * members]
    np.testing.assert_array_equal(out[:, :members], want_out[:, :members])
    np.testing.assert_array_equal(status, want_status)


def test_device_api_bounded_reports_deadlock(devapi):
    """Stripe 0 preset to 1 (not a multiple of its one member): the last round's
    target is never reached; the small poll bound ends it with DEADLOCK."""
    from cross_core_barrier_amd import ccb
    _say("device api soft_bounded, stripe 0 preset 1, 4x1x64, maxPoll 2000")
    st, _, _, status = _run(devapi, 3, 4, 1, 64, 0, 5, 1, max_poll=2000, preset=1)
    assert st == ccb.CCB_ERR_DEADLOCK
    assert (status == 3).any() and set(status.tolist()) <= {1, 3}


def test_device_api_rejects_bad_launch(devapi):
    """Refused before anything is launched (the launcher also refuses null
    buffers, which every case below passes)."""
    assert devapi.devapi_run(9, None, None, None, None, 0, 1, 1, 1, 64, 0, 0, None) != 0  # no variant 9
    assert devapi.devapi_run(6, None, None, None, None, 0, 1, 1, 1, 64, 0, 0, None) != 0  # null buffers
    assert devapi.devapi_run(5, None, None, None, None, 0, 1, 4, 1, 64, 2, 0, None) != 0  # 6 > 4
    assert devapi.devapi_run(0, None, None, None, None, 0, 1, 2, 1, 64, 3, 0, None) != 0
