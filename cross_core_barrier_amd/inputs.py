"""Seeded synthetic inputs shared by the GPU path's tests, the oracle's tests
and the benchmark.

This module draws random numbers and packs them into the boundary's input
layouts.  It holds none of the method's arithmetic: no counter update, no
predicate, no stencil, no barrier logic.  The mode codes it draws from are the
ones the CntNotify page enumerates ("CANN Runtime CntNotify（计数型通知）管理接口
详解", §3.1 record modes 0/1/2/4 and §3.2 wait modes 0-4).

Every generator uses numpy's default_rng(seed); workload k uses seed k.
"""

from __future__ import annotations

import hashlib
from typing import Tuple

import numpy as np

RECORD_CODES = np.array([0, 1, 2, 4], dtype=np.uint8)   # SET, ADD, OR, AND
WAIT_CODES = np.array([0, 1, 2, 3, 4], dtype=np.uint8)   # LESS, EQUAL, BIGGER, GE, BITMASK
ADD_CODE = 1

META_WAIT_BIT = 0x80
META_CLEAR_SHIFT = 3

# Workload shapes (seed = index).
WITNESS_SMALL = dict(seed=0, n_wg=8, threads=64, rounds=100)
WITNESS_GRID = dict(seed=1, n_wg=256, threads=256, rounds=10_000, used_cores_pass2=128)
STENCIL = dict(seed=2, n=1 << 26, iters=64, n_wg=1024, threads=256)
CNT_BATCH = dict(seed=3, n_counters=1 << 20, n_ops=64, wait_every=8)
GROUPED = dict(seed=4, n_wg=512, threads=256, rounds=100_000)


def encode_meta(mode: np.ndarray, is_wait: np.ndarray, is_clear: np.ndarray) -> np.ndarray:
    """Pack the per-op byte: bits 0-2 mode code, bit 3 isClear, bit 7 wait."""
    return (mode.astype(np.uint8)
            | (is_clear.astype(np.uint8) << META_CLEAR_SHIFT)
            | (is_wait.astype(np.uint8) * META_WAIT_BIT)).astype(np.uint8)


def stencil_input(seed: int, n: int, hi: int = 1 << 20) -> np.ndarray:
    """int32 values uniform in [0, hi)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, hi, size=n, dtype=np.int32)


def cnt_batch_input(seed: int, n_counters: int, n_ops: int, wait_every: int = 8,
                    small_values: bool = False) -> Tuple[np.ndarray, np.ndarray, int]:
    """Op-major (val uint32[n_ops, n_counters], meta uint8[n_ops, n_counters],
    number of wait rows).

    Op k is a wait when k % wait_every == wait_every - 1, a record otherwise.
    Records: mode uniform over {SET, ADD, OR, AND}; ADD values uniform in
    [0, 16), other values uniform over uint32.  Waits: mode uniform over the
    five wait codes, value uniform over uint32, isClear ~ Bernoulli(0.5).
    small_values=True draws every value from [0, 4) instead, so that EQUAL
    and BITMASK waits release often (directed coverage of those branches).
    """
    rng = np.random.default_rng(seed)
    shape = (n_ops, n_counters)
    k = np.arange(n_ops)[:, None]
    is_wait = np.broadcast_to((k % wait_every) == (wait_every - 1), shape)
    rec_mode = RECORD_CODES[rng.integers(0, len(RECORD_CODES), size=shape, dtype=np.uint8)]
    wait_mode = WAIT_CODES[rng.integers(0, len(WAIT_CODES), size=shape, dtype=np.uint8)]
    mode = np.where(is_wait, wait_mode, rec_mode)
    is_clear = is_wait & (rng.integers(0, 2, size=shape, dtype=np.uint8) == 1)
    if small_values:
        val = rng.integers(0, 4, size=shape, dtype=np.uint32)
    else:
        val = rng.integers(0, 1 << 32, size=shape, dtype=np.uint32)
        add_vals = rng.integers(0, 16, size=shape, dtype=np.uint32)
        val = np.where((~is_wait) & (mode == ADD_CODE), add_vals, val).astype(np.uint32)
    meta = encode_meta(mode, is_wait, is_clear)
    n_rel_rows = int(((np.arange(n_ops) % wait_every) == (wait_every - 1)).sum())
    return np.ascontiguousarray(val), np.ascontiguousarray(meta), n_rel_rows


# --- device-drawn inputs for sizes beyond a few GiB -------------------------
# The same recipes drawn by torch's generator on the device, where numpy would
# take minutes; seeded, so the same call gives the same tensor.

def stencil_input_device(seed: int, n: int, device="cuda", hi: int = 1 << 20):
    """int32 tensor of n values uniform in [0, hi), on the device."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(0, hi, (n,), generator=g, device=device, dtype=torch.int32)


def cnt_batch_input_device(seed: int, n_counters: int, n_ops: int, device="cuda",
                           wait_every: int = 8):
    """cnt_batch_input's recipe (without small_values) as device tensors:
    (val int32 bit patterns [n_ops, n_counters], meta uint8, wait rows)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (n_ops, n_counters)
    k = torch.arange(n_ops, device=device)[:, None]
    is_wait = ((k % wait_every) == (wait_every - 1)).expand(shape)
    rec = torch.as_tensor(RECORD_CODES, device=device)
    wt = torch.as_tensor(WAIT_CODES, device=device)
    rec_mode = rec[torch.randint(0, len(RECORD_CODES), shape, generator=g, device=device,
                                 dtype=torch.int32)]
    wait_mode = wt[torch.randint(0, len(WAIT_CODES), shape, generator=g, device=device,
                                 dtype=torch.int32)]
    mode = torch.where(is_wait, wait_mode, rec_mode)
    del rec_mode, wait_mode
    is_clear = is_wait & (torch.randint(0, 2, shape, generator=g, device=device,
                                        dtype=torch.uint8) == 1)
    val = torch.randint(0, 256, (n_ops, n_counters * 4), generator=g, device=device,
                        dtype=torch.uint8).view(torch.int32)
    add_vals = torch.randint(0, 16, shape, generator=g, device=device, dtype=torch.int32)
    val = torch.where((~is_wait) & (mode == ADD_CODE), add_vals, val)
    del add_vals
    meta = (mode | (is_clear.to(torch.uint8) << META_CLEAR_SHIFT)
            | (is_wait.to(torch.uint8) * META_WAIT_BIT)).to(torch.uint8)
    n_rel_rows = int(((np.arange(n_ops) % wait_every) == (wait_every - 1)).sum())
    return val.contiguous(), meta.contiguous(), n_rel_rows


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
