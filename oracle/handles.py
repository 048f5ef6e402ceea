"""Sequential model of the CntNotify handle life cycle and its error codes.

TEST INFRASTRUCTURE ONLY: part of the oracle.

Source: "CANN Runtime CntNotify（计数型通知）管理接口详解" (CANN Runtime CntNotify
interfaces):
  §3.3 record info {mode, value}; wait info {mode, value, timeout in seconds
       with 0 meaning forever, isClear, three reserved bytes};
  §4   every call returns 0 on success and an error code otherwise;
  §4.1 create: the flag is reserved and must be 0; creation fails when the
       notify resources run out;
  §4.2/§4.3 record and wait are asynchronous and reject a null info;
  §4.4 reset sets the count to 0 (asynchronous);
  §4.5 get-id rejects a null output pointer;
  §4.6 destroy releases the resource; the handle is unusable afterwards;
  §6.1 an invalid handle is reported as an error rather than crashing;
  §7   the clear of isClear happens after the wait has been released.

The model runs the device-side effects in one total order (the order in
which the GPU executes them).  A wait whose predicate is false stays pending
and is re-checked after every later record or reset, in order; a wait still
pending when the model is closed has timed out (finite timeout) or would
block forever (timeout 0).  This matches a polling GPU wait exactly when the
outcome does not depend on which intermediate counts the poll observes, which
is the only kind of sequence the tests give it.

Beyond the pages: abort(h) calls off the waits pending on h -- each ends
with CANCELLED and does not clear -- and leaves later waits alone (the
library's ccb_cnt_notify_abort; destroy does the same to the waits of the
handle it ends).

Status codes restated here (the oracle includes nothing from the library):
OK 0, INVALID_VALUE 1, NULL_POINTER 2, INVALID_HANDLE 3, RESOURCE_EXHAUSTED 4,
TIMEOUT 5, CANCELLED 11.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

OK, INVALID_VALUE, NULL_POINTER, INVALID_HANDLE, RESOURCE_EXHAUSTED, TIMEOUT = 0, 1, 2, 3, 4, 5
CANCELLED = 11

M32 = 0xFFFFFFFF


def record_op(count: int, mode: int, value: int) -> Optional[int]:
    """§3.1: 0 overwrite, 1 add (mod 2^32), 2 bit-or, 4 bit-and; else None."""
    if mode == 0:
        return value & M32
    if mode == 1:
        return (count + value) & M32
    if mode == 2:
        return count | value
    if mode == 4:
        return count & value
    return None


def wait_holds(count: int, mode: int, value: int) -> Optional[bool]:
    """§3.2: 0 less, 1 equal, 2 bigger, 3 bigger-or-equal, 4 (count & value) == value."""
    if mode == 0:
        return count < value
    if mode == 1:
        return count == value
    if mode == 2:
        return count > value
    if mode == 3:
        return count >= value
    if mode == 4:
        return (count & value) == value
    return None


@dataclass
class _Wait:
    mode: int
    value: int
    timeout_s: int
    is_clear: int
    outcome: Optional[int] = None  # OK once released


class CntNotifyModel:
    """Handles are small integers; capacity models the resource limit of §4.1."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.count: Dict[int, int] = {}
        self.pending: Dict[int, List[_Wait]] = {}
        self.last_wait: Dict[int, Optional[int]] = {}
        self.free_ids = list(range(capacity))

    # --- host-side calls -------------------------------------------------
    def create(self, flag: int) -> Tuple[int, Optional[int]]:
        if flag != 0:
            return INVALID_VALUE, None
        if not self.free_ids:
            return RESOURCE_EXHAUSTED, None
        h = self.free_ids.pop(0)
        self.count[h] = 0
        self.pending[h] = []
        self.last_wait[h] = None
        return OK, h

    def _valid(self, h) -> bool:
        return h is not None and h in self.count

    def record(self, h, info: Optional[Tuple[int, int]]) -> int:
        if not self._valid(h):
            return INVALID_HANDLE
        if info is None:
            return NULL_POINTER
        mode, value = info
        new = record_op(self.count[h], mode, value)
        if new is None:
            return INVALID_VALUE
        self.count[h] = new
        self._recheck(h)
        return OK

    def wait(self, h, info: Optional[Tuple[int, int, int, int]]) -> int:
        if not self._valid(h):
            return INVALID_HANDLE
        if info is None:
            return NULL_POINTER
        mode, value, timeout_s, is_clear = info
        if wait_holds(0, mode, value) is None or is_clear not in (0, 1):
            return INVALID_VALUE
        self.pending[h].append(_Wait(mode, value, timeout_s, is_clear))
        self._recheck(h)
        return OK

    def reset(self, h) -> int:
        if not self._valid(h):
            return INVALID_HANDLE
        self.count[h] = 0
        self._recheck(h)
        return OK

    def get_id(self, h, want_out: bool = True) -> Tuple[int, Optional[int]]:
        if not self._valid(h):
            return INVALID_HANDLE, None
        if not want_out:
            return NULL_POINTER, None
        return OK, h

    def abort(self, h) -> int:
        """Every wait pending on h ends with CANCELLED, without its clear."""
        if not self._valid(h):
            return INVALID_HANDLE
        if self.pending[h]:
            self.pending[h].clear()
            self.last_wait[h] = CANCELLED
        return OK

    def destroy(self, h) -> int:
        if not self._valid(h):
            return INVALID_HANDLE
        del self.count[h]
        del self.pending[h]
        del self.last_wait[h]
        self.free_ids.append(h)
        self.free_ids.sort()
        return OK

    # --- device-side progress -------------------------------------------
    def _recheck(self, h) -> None:
        """Release pending waits, in order, whose predicate now holds.  A
        stream blocks on its first pending wait, so waits release in FIFO
        order; the clear (isClear) follows the release."""
        q = self.pending[h]
        while q:
            w = q[0]
            if not wait_holds(self.count[h], w.mode, w.value):
                break
            w.outcome = OK
            self.last_wait[h] = OK
            if w.is_clear:
                self.count[h] = 0
            q.pop(0)

    def close(self, h) -> Optional[int]:
        """Finish: a wait still pending has timed out (or blocks forever when
        its timeout is 0, reported as None)."""
        q = self.pending[h]
        if q:
            w = q.pop(0)
            q.clear()
            if w.timeout_s == 0:
                self.last_wait[h] = None
                return None
            self.last_wait[h] = TIMEOUT
        return self.last_wait[h]
