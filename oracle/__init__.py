"""CPU oracle for the soft epoch barrier and CntNotify counter semantics.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the CPU
baseline leg of bench.py may import this package.  The product path (the
HIP library and its Python binding) never touches it, and it shares no code
with that path: the arithmetic lives in oracle/ccb_oracle.c (plain C, built
with gcc) and in the pure-Python enumerator and handle model beside it.
oracle/host_barrier.c runs the same arrival rule on host threads (a
concurrency check of the method and the CPU context figure).

Parity pins (what checks each oracle function against something other than
itself; see tests/test_oracle_*.py):

  witness_hash       SplitMix64 published output sequences (seed 0 and seed
                     1234567) -- pins the generator; the (seed, round, wg)
                     keying is this library's convention, not the pages'.
  mix_participants   the SYNCALL guide's §4.2 formula (blocks x (1 + ratio))
                     on its 1:1 and 1:2 cases, whole launch for 0.
  epoch_target,      the SYNCALL guide's §5.2 prose (next multiple of N above
  epoch_target_checked
                     the old count), checked by brute force over small
                     (before, N) against a search for that multiple.
  slot_rounds,       brute-force enumeration of every arrival order on small
  grouped_rounds     inputs (oracle/enumerate.py); closed forms for the
                     outputs (sum of members' witnesses) and the final
                     counters (rounds x members per counter).
  stencil            brute force over all inputs on n <= 4 with values < 4
                     against an independent numpy formulation, fixed points
                     (constants, x[i] = i in the interior), the max principle
                     and an exact mass identity.
  host_barrier       (not a reference for the GPU: the method on real host
                     threads) must reproduce slot_rounds' sums exactly.
  cnt_record,        the pages' mode tables (tests/golden), an exhaustive
  cnt_wait,          4-bit table against a set-of-bits restatement, 32-bit
  cnt_batch          edge cases (wrap, unsigned order), the pages' worked
                     examples, and identities (ADD 0, OR 0, AND ~0).

Nothing here is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ccb_oracle.c")
_SRC_HOST_BARRIER = os.path.join(_HERE, "host_barrier.c")
_LIB_PATH = os.path.join(_HERE, "libccb_oracle.so")
_lib = None

OK, INVALID_VALUE, DEADLOCK = 0, 1, 6


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into oracle/libccb_oracle.so."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < max(os.path.getmtime(_SRC),
                                              os.path.getmtime(_SRC_HOST_BARRIER)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, _SRC_HOST_BARRIER])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, u32, u64, i64 = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64
    lib.ccbo_splitmix64_nth.argtypes = [u64, u64]
    lib.ccbo_splitmix64_nth.restype = u64
    lib.ccbo_witness_hash.argtypes = [u64, u32, u32]
    lib.ccbo_witness_hash.restype = u32
    lib.ccbo_epoch_target.argtypes = [i32, i32]
    lib.ccbo_epoch_target.restype = i32
    lib.ccbo_epoch_target_checked.argtypes = [i32, i32, P]
    lib.ccbo_epoch_target_checked.restype = ctypes.c_int
    lib.ccbo_participants.argtypes = [i32, i32]
    lib.ccbo_participants.restype = i32
    lib.ccbo_mix_participants.argtypes = [i32, i32, i32]
    lib.ccbo_mix_participants.restype = i32
    lib.ccbo_slot_rounds.argtypes = [u64, i32, i32, i32, P, P, P]
    lib.ccbo_slot_rounds.restype = ctypes.c_int
    lib.ccbo_grouped_rounds.argtypes = [u64, i32, i32, P, P, P]
    lib.ccbo_grouped_rounds.restype = ctypes.c_int
    lib.ccbo_stencil.argtypes = [P, P, i64, i32]
    lib.ccbo_stencil.restype = None
    lib.ccbo_cnt_record.argtypes = [P, i32, u32]
    lib.ccbo_cnt_record.restype = ctypes.c_int
    lib.ccbo_cnt_wait_holds.argtypes = [u32, i32, u32, P]
    lib.ccbo_cnt_wait_holds.restype = ctypes.c_int
    lib.ccbo_cnt_wait_apply.argtypes = [P, i32, u32, i32, P]
    lib.ccbo_cnt_wait_apply.restype = ctypes.c_int
    lib.ccbo_cnt_batch.argtypes = [P, P, i64, i32, P, P, i32]
    lib.ccbo_cnt_batch.restype = ctypes.c_int
    lib.ccbo_host_barrier.argtypes = [i32, i32, u64, u64, P, ctypes.POINTER(ctypes.c_double)]
    lib.ccbo_host_barrier.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# --- witness hash / epoch ---------------------------------------------------

def splitmix64_nth(seed: int, n: int) -> int:
    return int(_load().ccbo_splitmix64_nth(seed, n))


def witness_hash(seed: int, rnd: int, wg: int) -> int:
    return int(_load().ccbo_witness_hash(seed, rnd, wg))


def epoch_target(before: int, n: int) -> int:
    return int(_load().ccbo_epoch_target(before, n))


def epoch_target_checked(before: int, n: int) -> Tuple[int, int]:
    """(rc, target): rc INVALID_VALUE when the target leaves the int32 range."""
    t = np.zeros(1, dtype=np.int32)
    rc = _load().ccbo_epoch_target_checked(before, n, _ptr(t))
    return int(rc), int(t[0])


def participants(used_cores: int, n_launched: int) -> int:
    return int(_load().ccbo_participants(used_cores, n_launched))


# --- round simulators -------------------------------------------------------

def slot_rounds(seed: int, rounds: int, n_grid: int, used_cores: int = 0,
                counter0: int = 0) -> Tuple[np.ndarray, np.ndarray, int, int]:
    """Witness rounds on one counter.  Returns (out[rounds, n_grid] uint32,
    status[n_grid] int32, final counter, rc)."""
    out = np.zeros((rounds, n_grid), dtype=np.uint32)
    status = np.zeros(n_grid, dtype=np.int32)
    ctr = np.array([counter0], dtype=np.int32)
    rc = _load().ccbo_slot_rounds(seed, rounds, n_grid, used_cores, _ptr(out), _ptr(status),
                                  _ptr(ctr))
    return out, status, int(ctr[0]), int(rc)


def mix_participants(groups: int, ratio: int, n_launched: int) -> int:
    return int(_load().ccbo_mix_participants(groups, ratio, n_launched))


def host_barrier(threads: int, rounds: int, seed: int, max_poll: int = 1 << 40
                 ) -> Tuple[np.ndarray, float, int]:
    """The flag-slot rounds on `threads` host threads through the epoch
    barrier.  Returns (out[rounds, threads] uint32, ns per barrier, rc)."""
    out = np.zeros((max(rounds, 0), max(threads, 1)), dtype=np.uint32)
    ns = ctypes.c_double(0.0)
    rc = _load().ccbo_host_barrier(threads, rounds, seed, max_poll, _ptr(out), ctypes.byref(ns))
    return out, float(ns.value), int(rc)


def grouped_rounds(seed: int, rounds: int, n_grid: int, counters0=(0, 0, 0)
                   ) -> Tuple[np.ndarray, np.ndarray, Tuple[int, int, int], int]:
    """Witness rounds over groups A (even), B (odd) and mix (all), round kind
    r mod 3.  Returns (out, status, (ctrA, ctrB, ctrMix), rc)."""
    out = np.zeros((rounds, n_grid), dtype=np.uint32)
    status = np.zeros(n_grid, dtype=np.int32)
    ctr = np.array(counters0, dtype=np.int32)
    rc = _load().ccbo_grouped_rounds(seed, rounds, n_grid, _ptr(out), _ptr(status), _ptr(ctr))
    return out, status, (int(ctr[0]), int(ctr[1]), int(ctr[2])), int(rc)


# --- stencil ----------------------------------------------------------------

def stencil(x: np.ndarray, iters: int) -> np.ndarray:
    """Returns the array after `iters` clamped 3-point iterations."""
    a = np.ascontiguousarray(x, dtype=np.int32).copy()
    b = np.empty_like(a)
    _load().ccbo_stencil(_ptr(a), _ptr(b), a.size, iters)
    return a if iters % 2 == 0 else b


# --- CntNotify ----------------------------------------------------------------

def cnt_record(count: int, mode: int, value: int) -> Tuple[int, int]:
    c = np.array([count], dtype=np.uint32)
    rc = _load().ccbo_cnt_record(_ptr(c), mode, value)
    return int(c[0]), int(rc)


def cnt_wait_holds(count: int, mode: int, value: int) -> Tuple[int, int]:
    h = np.zeros(1, dtype=np.int32)
    rc = _load().ccbo_cnt_wait_holds(count, mode, value, _ptr(h))
    return int(h[0]), int(rc)


def cnt_wait_apply(count: int, mode: int, value: int, is_clear: int) -> Tuple[int, int, int]:
    """Returns (new count, released, rc)."""
    c = np.array([count], dtype=np.uint32)
    rel = np.zeros(1, dtype=np.int32)
    rc = _load().ccbo_cnt_wait_apply(_ptr(c), mode, value, is_clear, _ptr(rel))
    return int(c[0]), int(rel[0]), int(rc)


def cnt_batch(val: np.ndarray, meta: np.ndarray, n_rel_rows: int
              ) -> Tuple[np.ndarray, np.ndarray, int]:
    """val uint32[nOps, nCounters], meta uint8[nOps, nCounters] (op-major).
    Returns (final uint32[nCounters], rel uint8[n_rel_rows, nCounters], rc)."""
    val = np.ascontiguousarray(val, dtype=np.uint32)
    meta = np.ascontiguousarray(meta, dtype=np.uint8)
    n_ops, n_counters = val.shape
    assert meta.shape == val.shape
    final = np.zeros(n_counters, dtype=np.uint32)
    rel = np.zeros((n_rel_rows, n_counters), dtype=np.uint8)
    rc = _load().ccbo_cnt_batch(_ptr(val), _ptr(meta), n_counters, n_ops, _ptr(final),
                                _ptr(rel), n_rel_rows)
    return final, rel, int(rc)
