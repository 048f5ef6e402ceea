"""The launchers' co-residency check against the hardware ([SYNCALL] §6.3:
every member of a persistent grid must be resident at once).  For each
workgroup size, the largest grid the launcher accepts (found by bisection;
a refused size launches nothing) must really run with every workgroup
resident: 20 barriers complete with a small poll bound instead of ending in
DEADLOCK, and every member arrives.  Workgroups whose wave count is not a
multiple of 4 are the shapes where an even spread over the SIMDs cannot be
assumed."""

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

THREADS = [64, 128, 192, 256, 320, 384, 448, 512, 640, 768, 1024]


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.fixture(scope="module")
def env():
    from cross_core_barrier_amd import ccb, workloads
    return ccb, workloads


def _largest(ccb, accept, hi):
    lo = 1
    while hi - lo > 1:
        mid = (lo + hi) // 2
        st = accept(mid)
        assert st in (ccb.CCB_OK, ccb.CCB_ERR_NOT_CORESIDENT), st
        torch.cuda.synchronize()
        if st == ccb.CCB_OK:
            lo = mid
        else:
            hi = mid
    return lo


@pytest.mark.parametrize("mode", [0, 2], ids=["striped-order", "striped-full"])
@pytest.mark.parametrize("threads", THREADS)
def test_barrier_only_accepted_grid_is_resident(env, threads, mode):
    ccb, wl = env
    n_cu = ccb.ccb_device_info()[1]
    n = _largest(ccb, lambda g: ccb.ccb_run_barrier_only(wl.workspace(1), None, None, 1, g,
                                                        threads, 0, 0, 0, mode, None), n_cu * 64)
    _say(f"barrier_only largest accepted grid {n}x{threads} ({n / n_cu:.2f} per CU), 20 rounds, "
         f"mode={mode}")
    ws = wl.workspace(1)
    assert ccb.ccb_run_barrier_only(ws, None, None, 20, n, threads, 0, 0, 200_000, mode, None) == 0
    st, ctrs = ccb.ccb_syncall_status(ws, 1, None)
    assert st == ccb.CCB_OK and ctrs == [20 * n]


@pytest.mark.parametrize("threads", THREADS)
def test_stencil_accepted_grid_is_resident(env, threads):
    ccb, wl = env
    n_cu = ccb.ccb_device_info()[1]
    a = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    b = torch.zeros_like(a)

    def accept(g):
        return ccb.ccb_run_stencil(a, b, a.numel(), 1, wl.workspace(1),
                                   wl.halo_scratch(a.numel(), threads, g), None, g, threads, 0, 0,
                                   0, None)
    n = _largest(ccb, accept, n_cu * 64)
    _say(f"stencil largest accepted grid {n}x{threads} ({n / n_cu:.2f} per CU), 20 iterations")
    ws = wl.workspace(1)
    halo = wl.halo_scratch(a.numel(), threads, n)
    assert ccb.ccb_run_stencil(a, b, a.numel(), 20, ws, halo, None, n, threads, 0, 200_000, 0,
                               None) == 0
    st, ctrs = ccb.ccb_syncall_status(ws, 1, None)
    assert st == ccb.CCB_OK and ctrs == [19 * n]
