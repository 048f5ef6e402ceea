"""ctypes binding of libccb.so (include/ccb.h), one Python function per C
entry point, with the same name.

Argument marshalling only: every step of the barrier, the stencil and the
CntNotify operations runs in the HIP kernels behind these calls.  Device
pointers may be given as ints or as torch tensors (their data_ptr()); streams
as ints (hipStream_t), torch.cuda.Stream objects, or None for the default
stream.  Each function returns the ccbStatus as an int; functions with output
parameters return (status, outputs...).

The library must have been built in-tree (python -m cross_core_barrier_amd.build);
if it is missing, importing this module raises -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libccb.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with `python -m cross_core_barrier_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

# status codes (include/ccb.h)
CCB_OK = 0
CCB_ERR_INVALID_VALUE = 1
CCB_ERR_NULL_POINTER = 2
CCB_ERR_INVALID_HANDLE = 3
CCB_ERR_RESOURCE_EXHAUSTED = 4
CCB_ERR_TIMEOUT = 5
CCB_ERR_DEADLOCK = 6
CCB_ERR_NOT_CORESIDENT = 7
CCB_ERR_UNSUPPORTED_DEVICE = 8
CCB_ERR_HIP = 9
CCB_ERR_NOT_READY = 10
CCB_ERR_CANCELLED = 11

CCB_SOFT_MAX_POLL = 1_000_000
CCB_BREAKDOWN_MAX_ROUNDS = 1024
CCB_NOALLOC_SCRATCH_BYTES = 4 << 20
CCB_LINE_BYTES = 128
CCB_STRIPES = 64
CCB_SLOT_ROWS = 6
CCB_SLOT_WORDS = 4
CCB_CNT_NOTIFY_POOL = 1024

CCB_BARRIER_STRIPED, CCB_BARRIER_FLAT, CCB_BARRIER_TREE = 0, 1, 4
CCB_VISIBILITY_ORDER, CCB_VISIBILITY_FULL, CCB_VISIBILITY_XCD = 0, 2, 8
CCB_TREE_GROUPS = 8
MODES = {
    "striped-order": CCB_BARRIER_STRIPED | CCB_VISIBILITY_ORDER,
    "striped-full": CCB_BARRIER_STRIPED | CCB_VISIBILITY_FULL,
    "striped-xcd": CCB_BARRIER_STRIPED | CCB_VISIBILITY_XCD,
    "flat-order": CCB_BARRIER_FLAT | CCB_VISIBILITY_ORDER,
    "flat-full": CCB_BARRIER_FLAT | CCB_VISIBILITY_FULL,
    "flat-xcd": CCB_BARRIER_FLAT | CCB_VISIBILITY_XCD,
    "tree-order": CCB_BARRIER_TREE | CCB_VISIBILITY_ORDER,
    "tree-full": CCB_BARRIER_TREE | CCB_VISIBILITY_FULL,
    "tree-xcd": CCB_BARRIER_TREE | CCB_VISIBILITY_XCD,
}
# word of a one-barrier workspace that holds the tree's top counter
CCB_TREE_TOP_WORD = (CCB_STRIPES - 1) * (CCB_LINE_BYTES // 4) + CCB_LINE_BYTES // 8
# words of a barrier's workspace that the per-XCD write-back uses: members
# registered per XCD, and the last round each XCD's leader wrote back
CCB_XCD_COUNT_WORD = 1 * (CCB_LINE_BYTES // 4) + 8
CCB_XCD_FLAG_WORD = 2 * (CCB_LINE_BYTES // 4) + 8

CCB_CNT_RECORD_SET_VALUE, CCB_CNT_RECORD_ADD, CCB_CNT_RECORD_BIT_OR, CCB_CNT_RECORD_BIT_AND = 0, 1, 2, 4
(CCB_CNT_WAIT_LESS, CCB_CNT_WAIT_EQUAL, CCB_CNT_WAIT_BIGGER, CCB_CNT_WAIT_BIGGER_OR_EQUAL,
 CCB_CNT_WAIT_EQUAL_WITH_BITMASK) = 0, 1, 2, 3, 4


class ccbCntRecordInfo(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("value", ctypes.c_uint32)]


class ccbCntWaitInfo(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("value", ctypes.c_uint32), ("timeout", ctypes.c_uint32),
                ("isClear", ctypes.c_uint8), ("rev", ctypes.c_uint8 * 3)]


class CcbError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {ccb_status_string(status)} ({status})")


def check(status: int, what: str = "ccb call") -> None:
    if status != CCB_OK:
        raise CcbError(status, what)


_V = ctypes.c_void_p
_I32, _U32, _I64, _U64 = ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_uint64


def _sig(name, restype, *argtypes):
    fn = getattr(_lib, name)
    fn.restype = restype
    fn.argtypes = list(argtypes)
    return fn


_f = {
    "ccb_status_string": _sig("ccb_status_string", ctypes.c_char_p, _I32),
    "ccb_version": _sig("ccb_version", _I32),
    "ccb_device_info": _sig("ccb_device_info", _I32, _V, _V, _V),
    "ccb_syncall_workspace_bytes": _sig("ccb_syncall_workspace_bytes", ctypes.c_size_t, _U32),
    "ccb_syncall_workspace_reset": _sig("ccb_syncall_workspace_reset", _I32, _V, _U32, _V),
    "ccb_syncall_status": _sig("ccb_syncall_status", _I32, _V, _U32, _V, _V),
    "ccb_run_barrier_only": _sig("ccb_run_barrier_only", _I32, _V, _V, _V, _I32, _I32, _I32, _I32,
                                 _I32, _U32, _I32, _V),
    "ccb_run_slot_rounds": _sig("ccb_run_slot_rounds", _I32, _V, _V, _V, _V, _U64, _I32, _I32, _I32,
                                _I32, _I32, _U32, _I32, _V),
    "ccb_run_grouped_rounds": _sig("ccb_run_grouped_rounds", _I32, _V, _V, _V, _V, _U64, _I32, _I32,
                                   _I32, _I32, _U32, _I32, _V),
    "ccb_bench_grouped_timeline": _sig("ccb_bench_grouped_timeline", _I32, _V, _V, _V, _V, _U64,
                                       _I32, _I32, _I32, _I32, _I32, _V),
    "ccb_run_stencil": _sig("ccb_run_stencil", _I32, _V, _V, _I64, _I32, _V, _V, ctypes.c_size_t,
                            _V, _I32, _I32, _I32, _U32, _I32, _V),
    "ccb_run_stencil_noalloc": _sig("ccb_run_stencil_noalloc", _I32, _V, _V, _I64, _I32, _V, _I32,
                                    _I32, _I32, _U32, _I32, _V),
    "ccb_stencil_halo_bytes": _sig("ccb_stencil_halo_bytes", ctypes.c_size_t, _I64, _I32, _I32),
    "ccb_bench_barrier_breakdown": _sig("ccb_bench_barrier_breakdown", _I32, _V, _V, _I32, _I32,
                                        _I32, _I32, _I32, _V),
    "ccb_bench_atomic_chain": _sig("ccb_bench_atomic_chain", _I32, _V, _V, _I32, _I32, _I32, _V),
    "ccb_bench_atomic_contended": _sig("ccb_bench_atomic_contended", _I32, _V, _V, _I32, _I32, _V),
    "ccb_bench_notify_pingpong": _sig("ccb_bench_notify_pingpong", _I32, _V, _V, _I32, _I32,
                                      _U32, _V, _V),
    "ccb_bench_fence_placement_bytes": _sig("ccb_bench_fence_placement_bytes", ctypes.c_size_t,
                                            _I32),
    "ccb_bench_fence_placement": _sig("ccb_bench_fence_placement", _I32, _V, ctypes.c_size_t, _V,
                                      _I32, _I32, _I32, _I32, _V),
    "ccb_bench_hip_grid_sync": _sig("ccb_bench_hip_grid_sync", _I32, _I32, _I32, _I32, _V, _V),
    "ccb_bench_copy": _sig("ccb_bench_copy", _I32, _V, _V, _I64, _V),
    "ccb_cnt_notify_create": _sig("ccb_cnt_notify_create", _I32, _V, _U64),
    "ccb_cnt_notify_record": _sig("ccb_cnt_notify_record", _I32, _V, _V, _V),
    "ccb_cnt_notify_wait": _sig("ccb_cnt_notify_wait", _I32, _V, _V, _V),
    "ccb_cnt_notify_reset": _sig("ccb_cnt_notify_reset", _I32, _V, _V),
    "ccb_cnt_notify_get_id": _sig("ccb_cnt_notify_get_id", _I32, _V, _V),
    "ccb_cnt_notify_destroy": _sig("ccb_cnt_notify_destroy", _I32, _V),
    "ccb_cnt_notify_abort": _sig("ccb_cnt_notify_abort", _I32, _V),
    "ccb_cnt_notify_query": _sig("ccb_cnt_notify_query", _I32, _V, _V, _V, _V),
    "ccb_cnt_notify_batch": _sig("ccb_cnt_notify_batch", _I32, _V, _V, _I64, _I32, _V, _V, _I32, _V,
                                 _V),
}

EXPORTED = sorted(_f)


def _p(x) -> Optional[int]:
    """Device pointer from an int, a torch tensor or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _s(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --- miscellaneous -------------------------------------------------------------

def ccb_status_string(s: int) -> str:
    return _f["ccb_status_string"](s).decode()


def ccb_version() -> int:
    return int(_f["ccb_version"]())


def ccb_device_info() -> Tuple[int, int, int, int]:
    cu, lds, clk = _I32(), _I32(), _I32()
    st = _f["ccb_device_info"](ctypes.byref(cu), ctypes.byref(lds), ctypes.byref(clk))
    return st, cu.value, lds.value, clk.value


# --- barrier ---------------------------------------------------------------------

def ccb_syncall_workspace_bytes(n_barriers: int) -> int:
    return int(_f["ccb_syncall_workspace_bytes"](n_barriers))


def ccb_syncall_workspace_reset(ws, n_barriers: int, stream=None) -> int:
    return _f["ccb_syncall_workspace_reset"](_p(ws), n_barriers, _s(stream))


def ccb_syncall_status(ws, n_barriers: int, stream=None):
    """Returns (status, [total arrivals per barrier])."""
    buf = (_I64 * max(n_barriers, 1))()
    st = _f["ccb_syncall_status"](_p(ws), n_barriers, buf, _s(stream))
    return st, [int(buf[i]) for i in range(n_barriers)]


def ccb_run_barrier_only(ws, placement, wg_status, rounds, n_grid, threads, used_cores=0,
                         wgs_per_cu=0, max_poll=0, mode=0, stream=None) -> int:
    return _f["ccb_run_barrier_only"](_p(ws), _p(placement), _p(wg_status), rounds, n_grid,
                                      threads, used_cores, wgs_per_cu, max_poll, mode, _s(stream))


def ccb_run_slot_rounds(ws, slots, out, wg_status, seed, rounds, n_grid, threads, used_cores=0,
                        wgs_per_cu=0, max_poll=0, mode=0, stream=None) -> int:
    return _f["ccb_run_slot_rounds"](_p(ws), _p(slots), _p(out), _p(wg_status), seed, rounds,
                                     n_grid, threads, used_cores, wgs_per_cu, max_poll, mode,
                                     _s(stream))


def ccb_run_grouped_rounds(ws, slots, out, wg_status, seed, rounds, n_grid, threads,
                           wgs_per_cu=0, max_poll=0, mode=0, stream=None) -> int:
    return _f["ccb_run_grouped_rounds"](_p(ws), _p(slots), _p(out), _p(wg_status), seed, rounds,
                                        n_grid, threads, wgs_per_cu, max_poll, mode, _s(stream))


def ccb_bench_grouped_timeline(ws, slots, out, stamps, seed, rounds, n_grid, threads,
                               wgs_per_cu=0, mode=0, stream=None) -> int:
    return _f["ccb_bench_grouped_timeline"](_p(ws), _p(slots), _p(out), _p(stamps), seed, rounds,
                                            n_grid, threads, wgs_per_cu, mode, _s(stream))


def ccb_stencil_halo_bytes(n: int, threads: int, n_grid: int) -> int:
    return int(_f["ccb_stencil_halo_bytes"](n, threads, n_grid))


def ccb_run_stencil(buf_a, buf_b, n, iters, ws, halo, halo_bytes, n_grid, threads, wgs_per_cu=0,
                    max_poll=0, mode=0, stream=None, timeline=None) -> int:
    """halo_bytes: size of the halo scratch; for a torch tensor pass None to
    use its size."""
    if halo_bytes is None:
        halo_bytes = 0 if halo is None else halo.numel() * halo.element_size()
    return _f["ccb_run_stencil"](_p(buf_a), _p(buf_b), n, iters, _p(ws), _p(halo), halo_bytes,
                                 _p(timeline), n_grid, threads, wgs_per_cu, max_poll, mode,
                                 _s(stream))


def ccb_run_stencil_noalloc(buf_a, buf_b, n, iters, status_out, n_grid, threads, wgs_per_cu=0,
                            max_poll=0, mode=0, stream=None) -> int:
    return _f["ccb_run_stencil_noalloc"](_p(buf_a), _p(buf_b), n, iters, _p(status_out), n_grid,
                                         threads, wgs_per_cu, max_poll, mode, _s(stream))


# --- floor microbenchmarks --------------------------------------------------------

def ccb_bench_barrier_breakdown(ws, stamps, rounds, n_grid, threads, wgs_per_cu=0, mode=0,
                                stream=None) -> int:
    return _f["ccb_bench_barrier_breakdown"](_p(ws), _p(stamps), rounds, n_grid, threads,
                                             wgs_per_cu, mode, _s(stream))


def ccb_bench_atomic_chain(line, ticks, iters, fenced=0, kind=0, stream=None) -> int:
    return _f["ccb_bench_atomic_chain"](_p(line), _p(ticks), iters, fenced, kind, _s(stream))


def ccb_bench_atomic_contended(line, ticks, iters, n_grid, stream=None) -> int:
    return _f["ccb_bench_atomic_contended"](_p(line), _p(ticks), iters, n_grid, _s(stream))


def ccb_bench_notify_pingpong(lines, ticks_out, iters, peer, max_poll, err, stream=None) -> int:
    return _f["ccb_bench_notify_pingpong"](_p(lines), _p(ticks_out), iters, peer, max_poll, _p(err),
                                           _s(stream))


def ccb_bench_fence_placement_bytes(n_grid: int) -> int:
    return int(_f["ccb_bench_fence_placement_bytes"](n_grid))


def ccb_bench_fence_placement(scratch, scratch_bytes, stale, rounds, n_grid, threads, variant,
                              stream=None) -> int:
    return _f["ccb_bench_fence_placement"](_p(scratch), scratch_bytes, _p(stale), rounds, n_grid,
                                           threads, variant, _s(stream))


def ccb_bench_hip_grid_sync(rounds, n_grid, threads, done_out, stream=None) -> int:
    return _f["ccb_bench_hip_grid_sync"](rounds, n_grid, threads, _p(done_out), _s(stream))


def ccb_bench_copy(dst, src, n_bytes, stream=None) -> int:
    return _f["ccb_bench_copy"](_p(dst), _p(src), n_bytes, _s(stream))


# --- CntNotify ----------------------------------------------------------------------

def ccb_cnt_notify_create(flag: int = 0, null_out: bool = False):
    """Returns (status, handle).  null_out=True passes a NULL out-pointer."""
    h = _V()
    st = _f["ccb_cnt_notify_create"](None if null_out else ctypes.byref(h), flag)
    return st, h.value


def ccb_cnt_notify_record(h, stream, info: Optional[ccbCntRecordInfo]) -> int:
    return _f["ccb_cnt_notify_record"](h, _s(stream), None if info is None else ctypes.byref(info))


def ccb_cnt_notify_wait(h, stream, info: Optional[ccbCntWaitInfo]) -> int:
    return _f["ccb_cnt_notify_wait"](h, _s(stream), None if info is None else ctypes.byref(info))


def ccb_cnt_notify_reset(h, stream=None) -> int:
    return _f["ccb_cnt_notify_reset"](h, _s(stream))


def ccb_cnt_notify_get_id(h, null_out: bool = False):
    i = _U32()
    st = _f["ccb_cnt_notify_get_id"](h, None if null_out else ctypes.byref(i))
    return st, i.value


def ccb_cnt_notify_destroy(h) -> int:
    return _f["ccb_cnt_notify_destroy"](h)


def ccb_cnt_notify_abort(h) -> int:
    return _f["ccb_cnt_notify_abort"](h)


def ccb_cnt_notify_query(h, stream=None):
    """Returns (status, value, last wait outcome)."""
    v, lw = _U32(), _I32()
    st = _f["ccb_cnt_notify_query"](h, ctypes.byref(v), ctypes.byref(lw), _s(stream))
    return st, v.value, lw.value


def ccb_cnt_notify_batch(val, meta, n_counters, n_ops, final, rel, n_rel_rows, err=None,
                         stream=None) -> int:
    return _f["ccb_cnt_notify_batch"](_p(val), _p(meta), n_counters, n_ops, _p(final), _p(rel),
                                      n_rel_rows, _p(err), _s(stream))


def record_info(mode: int, value: int) -> ccbCntRecordInfo:
    return ccbCntRecordInfo(mode, value & 0xFFFFFFFF)


def wait_info(mode: int, value: int, timeout: int = 0, is_clear: int = 0, rev=(0, 0, 0)) -> ccbCntWaitInfo:
    w = ccbCntWaitInfo(mode, value & 0xFFFFFFFF, timeout, is_clear)
    for i in range(3):
        w.rev[i] = rev[i]
    return w
