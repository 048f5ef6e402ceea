"""The entry points inside HIP graphs: each workload is captured once on a
stream and replayed several times, with eager work on the same buffers
between replays, and every replay is checked bit-exactly against the oracle.
Workspace resets are fill kernels, not memsets, so the graphs hold kernel
nodes only.  A first launch of each persistent kernel runs outside capture
(the launcher's one-time register queries synchronise)."""

import numpy as np
import pytest

import oracle
from cross_core_barrier_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.fixture(scope="module")
def env():
    from cross_core_barrier_amd import ccb, workloads
    # one eager launch of each persistent kernel before any capture
    workloads.barrier_only(2, 8, 64)
    workloads.slot_rounds(0, 2, 8, 64)
    workloads.grouped_rounds(4, 3, 8, 64)
    workloads.stencil(torch.zeros(4096, dtype=torch.int32, device="cuda"), 2, 4, 64)
    torch.cuda.synchronize()
    return ccb, workloads


@pytest.mark.parametrize("mode", [0, 8], ids=["striped-order", "striped-xcd"])
def test_graph_witness_rounds(env, mode):
    """Also with the per-XCD write-back, whose registration and flags live in
    the workspace: the captured reset clears them before every replay."""
    ccb, wl = env
    _say(f"graph: workspace reset + witness rounds 8x64, 100 rounds, 3 replays, mode={mode}")
    s = torch.cuda.Stream()
    ws = wl.workspace(1)
    slots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * 8, dtype=torch.int32, device="cuda")
    out = torch.zeros((100, 8), dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, s), "reset")
        ccb.check(ccb.ccb_run_slot_rounds(ws, slots, out, None, 0, 100, 8, 64, 0, 0, 0, mode, s),
                  "slot_rounds")
    want_out, _, want_ctr, rc = oracle.slot_rounds(0, 100, 8, 0)
    assert rc == 0
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        st, ctrs = ccb.ccb_syncall_status(ws, 1, None)
        assert st == 0 and ctrs == [want_ctr], (rep, st, ctrs)
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want_out)
        out.fill_(-1)  # eager work on the graph's buffers between replays
        ws.fill_(7)
        torch.cuda.synchronize()


def test_graph_stencil_and_grouped(env):
    ccb, wl = env
    _say("graph: input copy + stencil 50001 x 5 iterations, and grouped rounds 16x64, 30 rounds")
    s = torch.cuda.Stream()
    x = inputs.stencil_input(2, 50_001)
    x0 = torch.from_numpy(x).cuda()
    a, b = torch.empty_like(x0), torch.empty_like(x0)
    ws = wl.workspace(1)
    halo = wl.halo_scratch(x0.numel(), 128, 8)
    wsg = wl.workspace(3)
    slots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * 16, dtype=torch.int32, device="cuda")
    out = torch.zeros((30, 16), dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        a.copy_(x0)
        ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, s), "reset")
        ccb.check(ccb.ccb_run_stencil(a, b, a.numel(), 5, ws, halo, None, 8, 128, 0, 0, 0, s), "stencil")
        ccb.check(ccb.ccb_syncall_workspace_reset(wsg, 3, s), "reset 3")
        ccb.check(ccb.ccb_run_grouped_rounds(wsg, slots, out, None, 4, 30, 16, 64, 0, 0, 0, s), "grouped")
    want_y = oracle.stencil(x, 5)
    want_out, _, want_ctrs, rc = oracle.grouped_rounds(4, 30, 16)
    assert rc == 0
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert ccb.ccb_syncall_status(ws, 1, None)[0] == 0
        np.testing.assert_array_equal(b.cpu().numpy(), want_y)  # 5 iterations: the result is in b
        st, ctrs = ccb.ccb_syncall_status(wsg, 3, None)
        assert st == 0 and tuple(ctrs) == want_ctrs, (rep, st, ctrs)
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want_out)
        # grouped rounds leave a round's non-members' entries untouched, so
        # out is refilled with the zeros the oracle starts from
        a.fill_(3), b.fill_(3), out.zero_(), halo.fill_(9)
        torch.cuda.synchronize()


def test_graph_cntnotify(env):
    ccb, wl = env
    _say("graph: CntNotify record ADD 1 + wait GE 1 with clear, and a batch, 5 replays")
    s = torch.cuda.Stream()
    st, h = ccb.ccb_cnt_notify_create(0)
    assert st == 0
    val, meta, rows = inputs.cnt_batch_input(3, 1024, 16, small_values=True)
    v = torch.from_numpy(val.view(np.int32)).cuda()
    m = torch.from_numpy(meta).cuda()
    final = torch.empty(1024, dtype=torch.int32, device="cuda")
    rel = torch.zeros((rows, 1024), dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ccb.check(ccb.ccb_cnt_notify_record(h, s, ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 1)), "record")
        ccb.check(ccb.ccb_cnt_notify_wait(
            h, s, ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, 1, 2, 1)), "wait")
        ccb.check(ccb.ccb_cnt_notify_batch(v, m, 1024, 16, final, rel, rows, None, s), "batch")
    want_final, want_rel, rc = oracle.cnt_batch(val, meta, rows)
    assert rc == 0
    for rep in range(5):
        g.replay()
        torch.cuda.synchronize()
        assert ccb.ccb_cnt_notify_query(h, None) == (0, 0, ccb.CCB_OK), rep
        np.testing.assert_array_equal(final.cpu().numpy().view(np.uint32), want_final)
        np.testing.assert_array_equal(rel.cpu().numpy(), want_rel)
        final.fill_(-1), rel.fill_(2)
        torch.cuda.synchronize()
    assert ccb.ccb_cnt_notify_destroy(h) == 0
