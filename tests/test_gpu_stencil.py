"""GPU parity of the persistent barrier-separated stencil against the oracle
(bit-exact)."""

import numpy as np
import pytest

import oracle
from cross_core_barrier_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.fixture(scope="module")
def wl():
    from cross_core_barrier_amd import workloads
    return workloads


# striped / flat / tree x ordering-only / full fences / per-XCD write-back
MODES = [0, 1, 2, 3, 4, 6, 8, 9, 12]
MODE_IDS = ["striped-order", "flat-order", "striped-full", "flat-full", "tree-order", "tree-full",
            "striped-xcd", "flat-xcd", "tree-xcd"]


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("n,iters,n_grid,threads", [
    (1, 3, 1, 64),                 # single element
    (5, 4, 2, 64),                 # fewer elements than lanes
    (1000, 1, 3, 64),              # ragged spans, one iteration, no barrier
    (65536 * 3 + 17, 5, 16, 256),  # several full steps + ragged tail per wave
    (1 << 20, 8, 64, 256),         # several chunks per workgroup, no partial chunk
    (1024 * 5, 6, 7, 256),         # fewer chunks than workgroups
    (256 * 9 + 3, 9, 2, 64),       # partial last chunk after full ones, n % 4 != 0
    (1024 * 2000 + 5, 3, 1, 256),  # one workgroup, more chunks than the LDS staging holds
    (123457, 7, 37, 192),          # ragged everything, odd iteration count
    (4096, 0, 4, 64),              # zero iterations: result is the input
    (256 * 100, 10, 2, 64),        # one wave per workgroup
    (256 * 64 * 4, 7, 8, 256),     # all chunks full, several per workgroup
    (1024 * 3, 4, 5, 256),         # workgroups without chunks
    (1024 * 64, 2, 16, 1024),      # 1024-thread workgroups, two iterations
    # full chunks split evenly, 17 to 33 per workgroup
    (1024 * 17 * 4, 5, 4, 256),
    (256 * 20 * 3, 6, 3, 64),      # one wave per workgroup
    (1024 * 20, 4, 1, 256),        # a single workgroup
    (4096 * 18 * 2, 3, 2, 1024),   # 1024-thread workgroups
    (1024 * 33 * 8, 2, 8, 256),    # two iterations
])
def test_stencil_small(wl, n, iters, n_grid, threads, mode):
    _say(f"stencil mode={mode} n={n} iters={iters} grid={n_grid}x{threads}")
    x = inputs.stencil_input(2, n)
    st, y = wl.stencil(torch.from_numpy(x).cuda(), iters, n_grid, threads, mode=mode)
    assert st == 0
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.stencil(x, iters))


_full_cache = {}


@pytest.mark.parametrize("mode", [0, 2], ids=["striped-order", "striped-full"])
def test_stencil_full(wl, mode):
    """int32 x[2^26] uniform in [0, 2^20), 64 iterations, 1024 co-resident
    WGs x 256 threads (4 per CU), a barrier between iterations."""
    n = 1 << 26
    _say(f"stencil full n={n} iters=64 grid=1024x256 wgsPerCu=4 mode={mode}")
    x = inputs.stencil_input(2, n)
    st, y = wl.stencil(torch.from_numpy(x).cuda(), 64, 1024, 256, wgs_per_cu=4, mode=mode)
    assert st == 0
    if "want" not in _full_cache:
        _full_cache["want"] = oracle.stencil(x, 64)
    np.testing.assert_array_equal(y.cpu().numpy(), _full_cache["want"])


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_stencil_largest_coresident_grid(wl, mode):
    """1024-thread workgroups: the largest grid the launcher accepts (found by
    bisection; a refused size launches nothing) runs bit-exactly, and one
    workgroup more is refused."""
    from cross_core_barrier_amd import ccb
    a = torch.zeros(1024, dtype=torch.int32, device="cuda")
    b = torch.zeros_like(a)
    lo, hi = 1, 256 * 64
    while hi - lo > 1:
        mid = (lo + hi) // 2
        ws = wl.workspace(1)
        halo = wl.halo_scratch(1024, 1024, mid)
        st = ccb.ccb_run_stencil(a, b, 1024, 1, ws, halo, None, mid, 1024, 0, 0, mode, None)
        assert st in (ccb.CCB_OK, ccb.CCB_ERR_NOT_CORESIDENT)
        torch.cuda.synchronize()
        if st == ccb.CCB_OK:
            lo = mid
        else:
            hi = mid
    n, iters = 4096 * lo * 2 + 3, 3
    _say(f"stencil largest grid {lo}x1024 n={n} iters={iters} mode={mode}")
    x = inputs.stencil_input(21, n)
    st, y = wl.stencil(torch.from_numpy(x).cuda(), iters, lo, 1024, mode=mode)
    assert st == 0
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.stencil(x, iters))
    ws = wl.workspace(1)
    halo = wl.halo_scratch(1024, 1024, lo + 1)
    assert ccb.ccb_run_stencil(a, b, 1024, 1, ws, halo, None, lo + 1, 1024, 0, 0, mode, None) \
        == ccb.CCB_ERR_NOT_CORESIDENT


def test_stencil_invalid(wl):
    from cross_core_barrier_amd import ccb
    a = torch.zeros(1024, dtype=torch.int32, device="cuda")
    ws = wl.workspace(1)
    b = torch.zeros(1024, dtype=torch.int32, device="cuda")
    halo = wl.halo_scratch(1024, 64, 4)
    assert ccb.ccb_run_stencil(a, a, 1024, 1, ws, halo, None, 4, 64) == ccb.CCB_ERR_INVALID_VALUE  # overlap
    assert ccb.ccb_run_stencil(a.data_ptr() + 4, b, 100, 1, ws, halo, None, 4, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_stencil(a, None, 1024, 1, ws, halo, None, 4, 64) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_run_stencil(a, b, 1024, 1, ws, None, 0, 4, 64, mode=0) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_run_stencil(a, b, 1024, 1, ws, halo, None, 4, 64, mode=7) == ccb.CCB_ERR_INVALID_VALUE
    # scratch too small for the chunk count: rejected before launch
    assert ccb.ccb_run_stencil(a, b, 1024, 2, ws, halo, 16, 4, 64, mode=0) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_stencil(a, b, 1024, 2, ws, None, 0, 4, 64, mode=2) == ccb.CCB_OK
