"""Torch-side helpers around the C ABI: allocate device buffers with torch,
call the library, hand back tensors.  PyTorch provides memory and streams
only; every step of every workload runs in libccb.so's HIP kernels.

A helper given a stream (a torch.cuda.Stream or a raw hipStream_t) launches
on it after the buffers it filled on torch's current stream, and leaves the
current stream ordered after the launch.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import ccb

LINE_WORDS = ccb.CCB_LINE_BYTES // 4


def _dev(device) -> torch.device:
    return torch.device(device if device is not None else "cuda")


def _enter(stream, device):
    """Order a launch on `stream` after the allocations and fills this helper
    queued on torch's current stream.  Returns the stream as a torch stream
    (None for the default stream), for _leave."""
    if stream is None:
        return None
    s = stream if isinstance(stream, torch.cuda.Stream) else \
        torch.cuda.ExternalStream(int(stream), device=device)
    s.wait_stream(torch.cuda.current_stream(device))
    return s


def _leave(s, device) -> None:
    """Order torch's current stream after the launch, so that the returned
    tensors can be used there."""
    if s is not None:
        torch.cuda.current_stream(device).wait_stream(s)


def workspace(n_barriers: int, device=None) -> torch.Tensor:
    """A zeroed workspace for n_barriers barriers (their stripe lines plus
    the error line; int32, 128-B aligned)."""
    nbytes = ccb.ccb_syncall_workspace_bytes(n_barriers)
    ws = torch.zeros(nbytes // 4, dtype=torch.int32, device=_dev(device))
    if ws.data_ptr() % ccb.CCB_LINE_BYTES:
        raise RuntimeError("torch returned a workspace that is not 128-B aligned")
    return ws


@dataclass
class RoundsResult:
    status: int
    out: torch.Tensor          # uint32 [rounds, n_grid] (as int32 storage)
    wg_status: torch.Tensor    # int32 [n_grid]
    counters: list


def slot_rounds(seed: int, rounds: int, n_grid: int, threads: int, used_cores: int = 0,
                wgs_per_cu: int = 0, max_poll: int = 0, stream=None, device=None,
                out: Optional[torch.Tensor] = None, check_launch: bool = True,
                mode: int = 0) -> RoundsResult:
    d = _dev(device)
    ws = workspace(1, d)
    slots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * n_grid, dtype=torch.int32, device=d)
    if out is None:
        out = torch.zeros((rounds, n_grid), dtype=torch.int32, device=d)
    wg = torch.zeros(n_grid, dtype=torch.int32, device=d)
    s = _enter(stream, d)
    st = ccb.ccb_run_slot_rounds(ws, slots, out, wg, seed, rounds, n_grid, threads, used_cores,
                                 wgs_per_cu, max_poll, mode, stream)
    if check_launch:
        ccb.check(st, "ccb_run_slot_rounds")
    elif st != ccb.CCB_OK:
        return RoundsResult(st, out, wg, [])
    st, ctrs = ccb.ccb_syncall_status(ws, 1, stream)
    _leave(s, d)
    return RoundsResult(st, out, wg, ctrs)


def grouped_rounds(seed: int, rounds: int, n_grid: int, threads: int, wgs_per_cu: int = 0,
                   max_poll: int = 0, stream=None, device=None, mode: int = 0) -> RoundsResult:
    d = _dev(device)
    ws = workspace(3, d)
    slots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * n_grid, dtype=torch.int32, device=d)
    out = torch.zeros((rounds, n_grid), dtype=torch.int32, device=d)
    wg = torch.zeros(n_grid, dtype=torch.int32, device=d)
    s = _enter(stream, d)
    st = ccb.ccb_run_grouped_rounds(ws, slots, out, wg, seed, rounds, n_grid, threads, wgs_per_cu,
                                    max_poll, mode, stream)
    ccb.check(st, "ccb_run_grouped_rounds")
    st, ctrs = ccb.ccb_syncall_status(ws, 3, stream)
    _leave(s, d)
    return RoundsResult(st, out, wg, ctrs)


def barrier_only(rounds: int, n_grid: int, threads: int, used_cores: int = 0, wgs_per_cu: int = 0,
                 max_poll: int = 0, stream=None, device=None, placement: bool = False,
                 mode: int = 0):
    d = _dev(device)
    ws = workspace(1, d)
    wg = torch.zeros(n_grid, dtype=torch.int32, device=d)
    pl = torch.zeros(2 * n_grid, dtype=torch.int32, device=d) if placement else None
    s = _enter(stream, d)
    st = ccb.ccb_run_barrier_only(ws, pl, wg, rounds, n_grid, threads, used_cores, wgs_per_cu,
                                  max_poll, mode, stream)
    ccb.check(st, "ccb_run_barrier_only")
    st, ctrs = ccb.ccb_syncall_status(ws, 1, stream)
    _leave(s, d)
    return st, ctrs, wg, pl


def halo_scratch(n: int, threads: int, n_grid: int, device=None) -> torch.Tensor:
    nbytes = ccb.ccb_stencil_halo_bytes(n, threads, n_grid)
    return torch.zeros(max(nbytes // 4, 1), dtype=torch.int32, device=_dev(device))


def stencil(x: torch.Tensor, iters: int, n_grid: int, threads: int, wgs_per_cu: int = 0,
            max_poll: int = 0, stream=None, mode: int = 0):
    """Runs the persistent stencil on a copy of x; returns (status, result tensor)."""
    a = x.clone()
    b = torch.empty_like(a)
    ws = workspace(1, x.device)
    halo = halo_scratch(x.numel(), threads, n_grid, x.device)
    s = _enter(stream, x.device)
    st = ccb.ccb_run_stencil(a, b, a.numel(), iters, ws, halo, None, n_grid, threads, wgs_per_cu,
                             max_poll, mode, stream)
    ccb.check(st, "ccb_run_stencil")
    st, _ = ccb.ccb_syncall_status(ws, 1, stream)
    _leave(s, x.device)
    return st, (a if iters % 2 == 0 else b)


def cnt_batch(val: torch.Tensor, meta: torch.Tensor, n_rel_rows: int, stream=None):
    """val int32/uint32-bit-pattern [n_ops, n_counters], meta uint8 same shape.
    Returns (err word, final int32 [n_counters], rel uint8 [n_rel_rows, n_counters])."""
    n_ops, n_counters = val.shape
    final = torch.empty(n_counters, dtype=torch.int32, device=val.device)
    rel = torch.zeros((n_rel_rows, n_counters), dtype=torch.uint8, device=val.device)
    err = torch.zeros(1, dtype=torch.int32, device=val.device)
    s = _enter(stream, val.device)
    st = ccb.ccb_cnt_notify_batch(val, meta, n_counters, n_ops, final, rel, n_rel_rows, err, stream)
    ccb.check(st, "ccb_cnt_notify_batch")
    _leave(s, val.device)
    return err, final, rel
