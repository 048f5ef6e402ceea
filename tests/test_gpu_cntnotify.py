"""GPU parity of CntNotify: the batched engine against the oracle's
interpreter (bit-exact), and the stream-ordered handle API against the
pages' worked examples and the oracle's handle model."""

import numpy as np
import pytest

import oracle
from oracle import handles
from cross_core_barrier_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.fixture(scope="module")
def ccb():
    from cross_core_barrier_amd import ccb as lib
    return lib


@pytest.fixture(scope="module")
def wl(ccb):
    from cross_core_barrier_amd import workloads
    return workloads


def _run_batch(wl, val, meta, rows):
    v = torch.from_numpy(val.view(np.int32)).cuda()
    m = torch.from_numpy(meta).cuda()
    err, final, rel = wl.cnt_batch(v, m, rows)
    return int(err.item()), final.cpu().numpy().view(np.uint32), rel.cpu().numpy()


# --- batched engine -----------------------------------------------------------

@pytest.mark.parametrize("n_counters,n_ops,small", [
    (1024, 64, False), (1027, 64, False), (4096, 13, True), (4100, 64, True), (1, 8, True),
    (3, 0, False), (1026, 64, True), (2, 17, True),
])
def test_batch_small(wl, n_counters, n_ops, small):
    _say(f"cnt_batch n={n_counters} ops={n_ops} small_values={small}")
    val, meta, rows = inputs.cnt_batch_input(3, n_counters, n_ops, small_values=small)
    rows = max(rows, 1)
    err, final, rel = _run_batch(wl, val, meta, rows)
    f2, r2, rc = oracle.cnt_batch(val, meta, rows)
    assert rc == 0 and err == 0
    np.testing.assert_array_equal(final, f2)
    np.testing.assert_array_equal(rel, r2)


def test_batch_full(wl):
    """2^20 counters x 64 ops, a wait every 8th op."""
    _say("cnt_batch full n=2^20 ops=64")
    val, meta, rows = inputs.cnt_batch_input(3, 1 << 20, 64)
    err, final, rel = _run_batch(wl, val, meta, rows)
    f2, r2, rc = oracle.cnt_batch(val, meta, rows)
    assert rc == 0 and err == 0
    np.testing.assert_array_equal(final, f2)
    np.testing.assert_array_equal(rel, r2)


@pytest.mark.parametrize("n_counters", [8, 9])
def test_batch_malformed(wl, n_counters):
    _say(f"cnt_batch malformed ops n={n_counters}")
    val, meta, rows = inputs.cnt_batch_input(11, n_counters, 16, small_values=True)
    meta = meta.copy()
    meta[2, 1] = 3            # record code 3 does not exist
    meta[7, 2] |= 0x10        # reserved bit on a wait
    meta[4, 3] = 0x08         # isClear on a record
    meta[5, 4] = 0x80 | 6     # wait code 6 does not exist
    err, final, rel = _run_batch(wl, val, meta, rows)
    f2, r2, rc = oracle.cnt_batch(val, meta, rows)
    assert rc == oracle.INVALID_VALUE and err == oracle.INVALID_VALUE
    np.testing.assert_array_equal(final, f2)
    np.testing.assert_array_equal(rel, r2)


@pytest.mark.parametrize("n_counters", [4096, 4100, 4098])
def test_batch_malformed_in_uniform_rows(wl, n_counters):
    """Random op bytes (any code, clear and reserved bits) in 3% of the
    entries, keeping each op's wait bit, so that every op stays all-record or
    all-wait across the wave and malformed ops go through those rows' paths."""
    _say(f"cnt_batch random malformed ops in uniform rows n={n_counters}")
    val, meta, rows = inputs.cnt_batch_input(15, n_counters, 32, small_values=True)
    meta = meta.copy()
    rng = np.random.default_rng(16)
    hit = rng.random(meta.shape) < 0.03
    junk = rng.integers(0, 128, size=meta.shape).astype(np.uint8) | (meta & 0x80)
    meta[hit] = junk[hit]
    err, final, rel = _run_batch(wl, val, meta, rows)
    f2, r2, rc = oracle.cnt_batch(val, meta, rows)
    assert rc == oracle.INVALID_VALUE and err == oracle.INVALID_VALUE
    np.testing.assert_array_equal(final, f2)
    np.testing.assert_array_equal(rel, r2)


@pytest.mark.parametrize("n_counters", [4096, 4097])
def test_batch_waits_at_different_ops(wl, n_counters):
    """Each counter has its own wait positions, so neighbouring counters
    wait at different ops and their release flags land in different rows."""
    _say(f"cnt_batch per-counter wait positions n={n_counters}")
    n_ops = 48
    val, meta, _ = inputs.cnt_batch_input(13, n_counters, n_ops, small_values=True)
    meta = meta.copy()
    rng = np.random.default_rng(14)
    is_wait = rng.random((n_ops, n_counters)) < 0.2
    modes = rng.integers(0, 5, size=(n_ops, n_counters))
    clear = rng.random((n_ops, n_counters)) < 0.5
    wait_meta = (0x80 | modes | (clear.astype(np.int64) << 3)).astype(np.uint8)
    meta[is_wait] = wait_meta[is_wait]
    rec = (meta & 0x80) == 0
    meta[rec] = np.array([0, 1, 2, 4], np.uint8)[rng.integers(0, 4, size=rec.sum())]
    rows = int(((meta & 0x80) != 0).sum(axis=0).max())
    err, final, rel = _run_batch(wl, val, meta, rows)
    f2, r2, rc = oracle.cnt_batch(val, meta, rows)
    assert rc == 0 and err == 0
    np.testing.assert_array_equal(final, f2)
    np.testing.assert_array_equal(rel, r2)


def test_batch_too_few_rows(wl):
    val, meta, rows = inputs.cnt_batch_input(12, 64, 32, small_values=True)
    err, final, rel = _run_batch(wl, val, meta, rows - 1)
    f2, r2, rc = oracle.cnt_batch(val, meta, rows - 1)
    assert rc == err == oracle.INVALID_VALUE
    np.testing.assert_array_equal(final, f2)
    np.testing.assert_array_equal(rel, r2)


# --- stream-ordered handle API ---------------------------------------------------

def _mk(ccb):
    st, h = ccb.ccb_cnt_notify_create(0)
    assert st == 0
    return h


def test_worked_example_sec5(ccb):
    """CntNotify §5: stream 1 records ADD 1; stream 2 waits for >= 1 with a
    10 s timeout and clear-after-release; get the id; reset; destroy."""
    _say("cntnotify §5 example: record ADD 1 on s1, wait GE 1 clear on s2")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    h = _mk(ccb)
    assert ccb.ccb_cnt_notify_record(h, s1, ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 1)) == 0
    assert ccb.ccb_cnt_notify_wait(h, s2, ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, 1, 10, 1)) == 0
    st, v, last = ccb.ccb_cnt_notify_query(h, s2)
    assert (st, v, last) == (0, 0, ccb.CCB_OK)
    st, hid = ccb.ccb_cnt_notify_get_id(h)
    assert st == 0 and 0 <= hid < ccb.CCB_CNT_NOTIFY_POOL
    assert ccb.ccb_cnt_notify_reset(h, s2) == 0
    assert ccb.ccb_cnt_notify_query(h, s2)[:2] == (0, 0)
    assert ccb.ccb_cnt_notify_destroy(h) == 0


def test_n_producers(ccb):
    """CntNotify §5: N producer streams each record ADD 1; the consumer waits
    for >= N and is released only after all N."""
    n = 3
    _say(f"cntnotify {n} producers ADD 1, consumer GE {n}")
    prods = [torch.cuda.Stream() for _ in range(n)]
    cons = torch.cuda.Stream()
    h = _mk(ccb)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s in prods:
        assert ccb.ccb_cnt_notify_record(h, s, ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 1)) == 0
    assert ccb.ccb_cnt_notify_wait(h, cons, ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, n, 10, 0)) == 0
    with torch.cuda.stream(cons):
        flag.fill_(7)  # stream-ordered after the wait
    st, v, last = ccb.ccb_cnt_notify_query(h, cons)
    assert (st, v, last) == (0, n, ccb.CCB_OK)
    assert int(flag.item()) == 7
    assert ccb.ccb_cnt_notify_destroy(h) == 0


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16])
def test_n_producers_at_scale(ccb, n):
    """CntNotify §5 and §7 at scale: N producer streams (more streams than the
    process's hardware queues from N = 4 on) each record ADD 1 per round, the
    consumer stream waits GE N with isClear, over 100 rounds; every round is
    checked against the handle model.  The records are enqueued before the
    wait, so that no wait sits in a hardware queue in front of a record it
    needs (each producer first spins a little, so the wait usually starts
    polling before the records land)."""
    rounds = 100
    _say(f"cntnotify at scale: {n} producers ADD 1, consumer GE {n} with clear, {rounds} rounds")
    prods = [torch.cuda.Stream() for _ in range(n)]
    cons = torch.cuda.Stream()
    h = _mk(ccb)
    m = handles.CntNotifyModel(capacity=1)
    _, mh = m.create(0)
    for r in range(rounds):
        for s in prods:
            with torch.cuda.stream(s):
                torch.cuda._sleep(20000)
            assert ccb.ccb_cnt_notify_record(h, s, ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 1)) == 0
            assert m.record(mh, (ccb.CCB_CNT_RECORD_ADD, 1)) == handles.OK
        assert ccb.ccb_cnt_notify_wait(
            h, cons, ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, n, 2, 1)) == 0
        assert m.wait(mh, (ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, n, 2, 1)) == handles.OK
        torch.cuda.synchronize()
        st, v, last = ccb.ccb_cnt_notify_query(h, cons)
        assert (st, v, last) == (0, m.count[mh], m.last_wait[mh]) == (0, 0, ccb.CCB_OK), r
    assert ccb.ccb_cnt_notify_destroy(h) == 0


def test_abort_ends_a_pending_wait(ccb):
    """ccb_cnt_notify_abort from the host while a wait (GE 1, nothing will
    record) polls: the wait ends with CANCELLED well before its 5 s limit,
    does not clear, and the handle keeps working; as in the handle model."""
    import time
    _say("cntnotify abort of a polling wait (5 s limit, no record)")
    s = torch.cuda.Stream()
    h = _mk(ccb)
    m = handles.CntNotifyModel(capacity=1)
    _, mh = m.create(0)
    assert ccb.ccb_cnt_notify_record(h, s, ccb.record_info(ccb.CCB_CNT_RECORD_SET_VALUE, 0)) == 0
    m.record(mh, (ccb.CCB_CNT_RECORD_SET_VALUE, 0))
    t0 = time.perf_counter()
    assert ccb.ccb_cnt_notify_wait(h, s, ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, 1, 5, 1)) == 0
    m.wait(mh, (ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, 1, 5, 1))
    time.sleep(0.05)  # the wait is polling by now
    assert ccb.ccb_cnt_notify_abort(h) == 0
    m.abort(mh)
    s.synchronize()
    assert time.perf_counter() - t0 < 2.0
    st, v, last = ccb.ccb_cnt_notify_query(h, s)
    assert (st, v, last) == (0, m.count[mh], m.last_wait[mh]) == (0, 0, ccb.CCB_ERR_CANCELLED)
    # later waits are not affected
    assert ccb.ccb_cnt_notify_record(h, s, ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 4)) == 0
    assert ccb.ccb_cnt_notify_wait(h, s, ccb.wait_info(ccb.CCB_CNT_WAIT_EQUAL, 4, 5, 1)) == 0
    assert ccb.ccb_cnt_notify_query(h, s) == (0, 0, ccb.CCB_OK)
    assert ccb.ccb_cnt_notify_destroy(h) == 0
    assert ccb.ccb_cnt_notify_abort(h) == ccb.CCB_ERR_INVALID_HANDLE


def test_destroy_ends_a_pending_wait(ccb):
    """A wait still polling when its handle is destroyed ends (CANCELLED), so
    its stream does not stay blocked until the 5 s limit."""
    import time
    _say("cntnotify destroy while a wait polls (5 s limit, no record)")
    s = torch.cuda.Stream()
    h = _mk(ccb)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    t0 = time.perf_counter()
    assert ccb.ccb_cnt_notify_wait(h, s, ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, 1, 5, 0)) == 0
    with torch.cuda.stream(s):
        flag.fill_(1)  # ordered after the wait
    time.sleep(0.05)
    assert ccb.ccb_cnt_notify_destroy(h) == 0
    s.synchronize()
    assert time.perf_counter() - t0 < 2.0
    assert int(flag.item()) == 1


def test_stale_record_does_not_reach_the_next_owner(ccb):
    """A record enqueued for a handle, but run only after that handle was
    destroyed and its line given to a new handle, changes the old
    generation's count, not the new owner's."""
    _say("cntnotify stale record after the line changed owner")
    hs = []
    for _ in range(ccb.CCB_CNT_NOTIFY_POOL):
        st, x = ccb.ccb_cnt_notify_create(0)
        assert st == 0
        hs.append(x)
    old = hs.pop(7)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(20_000_000)  # the record below runs after the re-create
    assert ccb.ccb_cnt_notify_record(old, s, ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 5)) == 0
    line = ccb.ccb_cnt_notify_get_id(old)[1]
    assert ccb.ccb_cnt_notify_destroy(old) == 0
    st, new = ccb.ccb_cnt_notify_create(0)  # the only free line: the same one
    assert st == 0 and ccb.ccb_cnt_notify_get_id(new)[1] == line
    hs.append(new)
    s.synchronize()
    assert ccb.ccb_cnt_notify_query(new, None) == (0, 0, ccb.CCB_ERR_NOT_READY)
    for x in hs:
        assert ccb.ccb_cnt_notify_destroy(x) == 0


def test_rounds_reuse_with_clear(ccb):
    """CntNotify §5/§7: the same counter reused round after round -- N producer
    streams ADD 1, the consumer waits GE N with isClear -- each round released
    and cleared back to 0 (rounds separated on the host, as a real producer
    would wait for the consumer before its next record)."""
    n, rounds = 2, 20
    _say(f"cntnotify {rounds} rounds: {n} producers ADD 1, consumer GE {n} with clear")
    prods = [torch.cuda.Stream() for _ in range(n)]
    cons = torch.cuda.Stream()
    h = _mk(ccb)
    for r in range(rounds):
        # producers first: a wait never sits in a hardware queue in front of
        # the records it waits for; their short spin lets the wait start first
        for s in prods:
            with torch.cuda.stream(s):
                torch.cuda._sleep(50000)
            assert ccb.ccb_cnt_notify_record(h, s, ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 1)) == 0
        assert ccb.ccb_cnt_notify_wait(
            h, cons, ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, n, 2, 1)) == 0
        torch.cuda.synchronize()
        st, v, last = ccb.ccb_cnt_notify_query(h, cons)
        assert (st, v, last) == (0, 0, ccb.CCB_OK), r
    assert ccb.ccb_cnt_notify_destroy(h) == 0


def test_wait_timeout(ccb):
    _say("cntnotify wait GE 5 with 1 s timeout and no record: expect TIMEOUT")
    s = torch.cuda.Stream()
    h = _mk(ccb)
    assert ccb.ccb_cnt_notify_record(h, s, ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 2)) == 0
    assert ccb.ccb_cnt_notify_wait(h, s, ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, 5, 1, 1)) == 0
    st, v, last = ccb.ccb_cnt_notify_query(h, s)
    assert (st, v, last) == (0, 2, ccb.CCB_ERR_TIMEOUT)  # timed out: no clear
    assert ccb.ccb_cnt_notify_destroy(h) == 0


def test_record_modes_vs_model(ccb):
    """A sequence of every record mode and released waits on one stream,
    checked against the oracle's handle model after each step."""
    _say("cntnotify mode sequence on one stream vs handle model")
    s = torch.cuda.Stream()
    h = _mk(ccb)
    m = handles.CntNotifyModel(capacity=1)
    _, mh = m.create(0)
    seq = [("rec", 0, 0xF0F0), ("rec", 1, 0x0F), ("rec", 2, 0x100), ("rec", 4, 0xFF0F),
           ("wait", 4, 0x010F, 1, 0), ("rec", 1, 0xFFFFFFFF), ("wait", 2, 0, 1, 1),
           ("rec", 0, 7), ("wait", 1, 7, 1, 0), ("rec", 4, 3), ("wait", 0, 4, 1, 1)]
    for op in seq:
        if op[0] == "rec":
            assert ccb.ccb_cnt_notify_record(h, s, ccb.record_info(op[1], op[2])) == 0
            assert m.record(mh, (op[1], op[2])) == 0
        else:
            assert ccb.ccb_cnt_notify_wait(h, s, ccb.wait_info(op[1], op[2], op[3], op[4])) == 0
            assert m.wait(mh, (op[1], op[2], op[3], op[4])) == 0
            assert m.last_wait[mh] == handles.OK, op  # every wait here releases
        st, v, last = ccb.ccb_cnt_notify_query(h, s)
        assert st == 0 and v == m.count[mh], op
    assert ccb.ccb_cnt_notify_destroy(h) == 0


def test_handle_errors_and_pool(ccb):
    _say("cntnotify handle errors and pool exhaustion")
    assert ccb.ccb_cnt_notify_create(1)[0] == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_cnt_notify_create(0, null_out=True)[0] == ccb.CCB_ERR_NULL_POINTER
    h = _mk(ccb)
    assert ccb.ccb_cnt_notify_record(h, None, None) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_cnt_notify_wait(h, None, None) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_cnt_notify_record(h, None, ccb.record_info(3, 1)) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_cnt_notify_wait(h, None, ccb.wait_info(5, 1, 1)) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_cnt_notify_wait(h, None, ccb.wait_info(3, 1, 1, 2)) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_cnt_notify_wait(h, None, ccb.wait_info(3, 1, 1, 0, (0, 1, 0))) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_cnt_notify_get_id(h, null_out=True)[0] == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_cnt_notify_destroy(h) == 0
    assert ccb.ccb_cnt_notify_destroy(h) == ccb.CCB_ERR_INVALID_HANDLE
    assert ccb.ccb_cnt_notify_record(h, None, ccb.record_info(1, 1)) == ccb.CCB_ERR_INVALID_HANDLE
    assert ccb.ccb_cnt_notify_reset(h, None) == ccb.CCB_ERR_INVALID_HANDLE
    assert ccb.ccb_cnt_notify_get_id(0x12345)[0] == ccb.CCB_ERR_INVALID_HANDLE
    hs = []
    for _ in range(ccb.CCB_CNT_NOTIFY_POOL):
        st, hh = ccb.ccb_cnt_notify_create(0)
        assert st == 0
        hs.append(hh)
    assert ccb.ccb_cnt_notify_create(0)[0] == ccb.CCB_ERR_RESOURCE_EXHAUSTED
    ids = {ccb.ccb_cnt_notify_get_id(x)[1] for x in hs}
    assert len(ids) == ccb.CCB_CNT_NOTIFY_POOL
    assert ccb.ccb_cnt_notify_destroy(hs[5]) == 0
    st, again = ccb.ccb_cnt_notify_create(0)
    assert st == 0 and again != hs[5]               # same line, new generation
    assert ccb.ccb_cnt_notify_record(hs[5], None, ccb.record_info(1, 1)) == ccb.CCB_ERR_INVALID_HANDLE
    hs[5] = again
    for x in hs:
        assert ccb.ccb_cnt_notify_destroy(x) == 0


def test_handle_table_under_threads(ccb):
    """The handle table is shared by host threads ([CNTNOTIFY] §6.1: a handle
    is either valid or an error): threads that create at once get distinct
    lines, and of threads that destroy one handle at once exactly one
    succeeds."""
    import threading
    _say("cntnotify handle table from 8 host threads")
    torch.cuda.init()
    made, lock = [], threading.Lock()

    def create(k):
        torch.cuda.set_device(0)
        for _ in range(k):
            st, h = ccb.ccb_cnt_notify_create(0)
            assert st == 0
            with lock:
                made.append(h)

    ts = [threading.Thread(target=create, args=(64,)) for _ in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert len(made) == 512
    assert len({ccb.ccb_cnt_notify_get_id(h)[1] for h in made}) == 512
    outcomes = []
    go = threading.Barrier(8)

    def destroy(h):
        torch.cuda.set_device(0)
        go.wait()
        outcomes.append(ccb.ccb_cnt_notify_destroy(h))

    for h in made[:16]:
        outcomes.clear()
        ts = [threading.Thread(target=destroy, args=(h,)) for _ in range(8)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        assert sorted(outcomes) == [0] + [ccb.CCB_ERR_INVALID_HANDLE] * 7
    for h in made[16:]:
        assert ccb.ccb_cnt_notify_destroy(h) == 0


def test_wait_without_limit_already_satisfied(ccb):
    """timeout 0 means no limit ([CNTNOTIFY] §4.3); a wait whose predicate
    already holds when it starts is released at once, with its clear.  (The
    record is complete before the wait is enqueued, so the wait cannot be
    left waiting.)"""
    _say("cntnotify wait with no time limit, predicate already true")
    h = _mk(ccb)
    s = torch.cuda.Stream()
    assert ccb.ccb_cnt_notify_record(h, s, ccb.record_info(ccb.CCB_CNT_RECORD_SET_VALUE, 5)) == 0
    torch.cuda.synchronize()
    assert ccb.ccb_cnt_notify_wait(h, s, ccb.wait_info(ccb.CCB_CNT_WAIT_EQUAL, 5, 0, 1)) == 0
    assert ccb.ccb_cnt_notify_query(h, s) == (0, 0, ccb.CCB_OK)
    assert ccb.ccb_cnt_notify_destroy(h) == 0
