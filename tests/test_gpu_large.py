"""Parity where 32-bit offsets would overflow: a stencil array of more than
2^31 int32 (8 GiB per buffer) and a CntNotify batch whose operand array is
larger than 4 GiB.  Outputs are sampled and the oracle computes each sample
from the same inputs: a stencil output after T iterations depends only on the
inputs within distance T (checked on the CPU below), and batch counters are
independent, so a subset of columns is a batch of its own."""

import numpy as np
import pytest

import oracle
from cross_core_barrier_amd import inputs

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


def _stencil_samples(x_at, n, iters, pos):
    """Oracle values of the stencil output at positions pos after `iters`
    iterations.  x_at(idx) returns the input at the int64 indices idx.  Each
    sample runs the oracle on the window of half-width iters + 2 around it,
    cut at the array ends (where the window's own clamping is the array's)."""
    h = iters + 2
    lo = np.maximum(pos - h, 0)
    hi = np.minimum(pos + h + 1, n)
    offs = [np.arange(a, b, dtype=np.int64) for a, b in zip(lo, hi)]
    vals = x_at(np.concatenate(offs))
    out, k = np.empty(len(pos), dtype=np.int32), 0
    for i, (p, a, o) in enumerate(zip(pos, lo, offs)):
        window = vals[k:k + len(o)]
        k += len(o)
        out[i] = oracle.stencil(window, iters)[p - a]
    return out


def test_stencil_window_sampling_matches_full_oracle():
    """The sampling above gives the full oracle's value at every position,
    ends included (CPU)."""
    for n, iters in ((50, 3), (13, 5), (200, 1), (7, 0)):
        x = inputs.stencil_input(9, n)
        pos = np.arange(n, dtype=np.int64)
        got = _stencil_samples(lambda idx: x[idx], n, iters, pos)
        np.testing.assert_array_equal(got, oracle.stencil(x, iters))


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [0, 2], ids=["striped-order", "striped-full"])
def test_stencil_beyond_int32_offsets(mode):
    from cross_core_barrier_amd import workloads as wl
    n, iters = (1 << 31) + 1027, 3  # partial last chunk; n % 4 == 3
    _say(f"stencil large n={n} iters={iters} grid=1024x256 wgsPerCu=4 mode={mode}")
    x = inputs.stencil_input_device(12, n)
    rng = np.random.default_rng(12)
    b31 = 1 << 31
    pos = np.unique(np.concatenate([
        np.arange(0, 9), np.arange(n - 9, n), np.arange(b31 - 8, b31 + 9),
        np.arange((1 << 30) - 4, (1 << 30) + 5),
        np.array([c * 1024 + d for c in (2097151, 2097152, 2097153) for d in (-1, 0, 1)]),
        rng.integers(0, n, 2000)]).astype(np.int64))
    want = _stencil_samples(
        lambda idx: x[torch.from_numpy(idx).cuda()].cpu().numpy(), n, iters, pos)
    st, y = wl.stencil(x, iters, 1024, 256, wgs_per_cu=4, mode=mode)
    assert st == 0
    del x
    got = y[torch.from_numpy(pos).cuda()].cpu().numpy()
    np.testing.assert_array_equal(got, want)
    del y
    torch.cuda.empty_cache()


@pytest.mark.gpu
@pytest.mark.parametrize("n_counters", [1 << 27, (1 << 27) + 1],
                         ids=["vector", "one-per-lane"])
def test_batch_beyond_4GiB(n_counters):
    from cross_core_barrier_amd import workloads as wl
    n_ops = 9  # op 8 of every counter lies past byte 2^32 of val
    _say(f"cnt batch large n_counters={n_counters} n_ops={n_ops}")
    val, meta, rows = inputs.cnt_batch_input_device(13, n_counters, n_ops)
    assert val.numel() * 4 > (1 << 32)
    rng = np.random.default_rng(13)
    cols = np.unique(np.concatenate([
        np.arange(0, 64), np.arange(n_counters - 64, n_counters),
        rng.integers(0, n_counters, 4096)]).astype(np.int64))
    ci = torch.from_numpy(cols).cuda()
    v_s = val[:, ci].cpu().numpy().view(np.uint32)
    m_s = meta[:, ci].cpu().numpy()
    err, final, rel = wl.cnt_batch(val, meta, rows)
    del val, meta
    want_final, want_rel, rc = oracle.cnt_batch(np.ascontiguousarray(v_s),
                                                np.ascontiguousarray(m_s), rows)
    assert rc == 0 and int(err.item()) == 0
    np.testing.assert_array_equal(final[ci].cpu().numpy().view(np.uint32),
                                  want_final.view(np.uint32))
    np.testing.assert_array_equal(rel[:, ci].cpu().numpy(), want_rel)
    del final, rel
    torch.cuda.empty_cache()
