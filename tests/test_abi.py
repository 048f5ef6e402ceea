"""The C ABI on the CPU: the library loads, exports every entry point the
headers declare, its structs have the documented layout, its constants match
the pages' tables, and argument validation that precedes any device work
returns the documented codes.  No compute call is made here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _declared():
    names = set()
    for fn in sorted(os.listdir(INCLUDE)):
        if fn.endswith(".h"):
            text = open(os.path.join(INCLUDE, fn)).read()
            names |= set(re.findall(r"CCB_API\s+[\w\s\*]+?\b(ccb_\w+)\s*\(", text))
    return names


def _header_enum(name_prefix):
    text = open(os.path.join(INCLUDE, "ccb.h")).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(rf"\b({name_prefix}\w*)\s*=\s*(\d+)", text)}


@pytest.fixture(scope="module")
def ccb():
    from cross_core_barrier_amd import ccb as lib
    return lib


def test_library_exports_every_declared_symbol(ccb):
    lib = ctypes.CDLL(ccb.LIB_PATH)
    declared = _declared()
    assert len(declared) >= 20
    missing = [n for n in sorted(declared) if not hasattr(lib, n)]
    assert missing == []
    assert set(ccb.EXPORTED) == declared


def test_struct_layouts(ccb):
    assert ctypes.sizeof(ccb.ccbCntRecordInfo) == 8
    assert ctypes.sizeof(ccb.ccbCntWaitInfo) == 16
    assert ccb.ccbCntWaitInfo.isClear.offset == 12
    assert ccb.ccbCntWaitInfo.rev.offset == 13


def _golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                code, label, _ = line.split()
                rows[label] = int(code)
    return rows


def test_mode_codes_match_pages():
    rec = _header_enum("CCB_CNT_RECORD_")
    wait = _header_enum("CCB_CNT_WAIT_")
    assert {k[len("CCB_CNT_RECORD_"):]: v for k, v in rec.items()} == _golden("cntnotify_record_modes.txt")
    assert {k[len("CCB_CNT_WAIT_"):]: v for k, v in wait.items()} == _golden("cntnotify_wait_modes.txt")


def test_status_codes_consistent(ccb):
    hdr = _header_enum("CCB_ERR_")
    for name, val in hdr.items():
        assert getattr(ccb, name) == val
        assert ccb.ccb_status_string(val) == name
    assert ccb.ccb_status_string(0) == "CCB_OK"
    assert ccb.ccb_version() >= 100


def test_constants_match_pages(ccb):
    consts = {}
    with open(os.path.join(GOLDEN, "syncall_constants.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                consts[k] = int(v)
    text = open(os.path.join(INCLUDE, "ccb.h")).read()
    m = re.search(r"#define CCB_SOFT_MAX_POLL (\d+)u", text)
    assert int(m.group(1)) == consts["soft_max_poll_iterations"] == ccb.CCB_SOFT_MAX_POLL
    # every numeric constant of the header that the binding mirrors
    defines = {m.group(1): int(m.group(2))
               for m in re.finditer(r"#define (CCB_\w+) (\d+)u?\s*$", text, re.M)}
    enums = {**_header_enum("CCB_BARRIER_"), **_header_enum("CCB_VISIBILITY_"),
             **_header_enum("CCB_CNT_RECORD_"), **_header_enum("CCB_CNT_WAIT_")}
    for name in ("CCB_STRIPES", "CCB_SLOT_ROWS", "CCB_SLOT_WORDS", "CCB_LINE_BYTES",
                 "CCB_CNT_NOTIFY_POOL", "CCB_SOFT_MAX_POLL", "CCB_TREE_GROUPS",
                 "CCB_BREAKDOWN_MAX_ROUNDS"):
        assert defines.get(name) == getattr(ccb, name), name
    assert len(enums) == 15
    for name, val in enums.items():
        assert getattr(ccb, name) == val, name
    assert ccb.MODES == {"striped-order": 0, "flat-order": 1, "striped-full": 2, "flat-full": 3,
                         "tree-order": 4, "tree-full": 6, "striped-xcd": 8, "flat-xcd": 9,
                         "tree-xcd": 12}
    # the per-XCD bookkeeping words of the device header, as the binding has them
    dev = open(os.path.join(INCLUDE, "ccb_device.h")).read()
    for name in ("CCB_XCD_COUNT_WORD", "CCB_XCD_FLAG_WORD"):
        expr = re.search(r"#define %s \((.*)\)" % name, dev).group(1)
        value = eval(expr.replace("CCB_LINE_WORDS", str(ccb.CCB_LINE_BYTES // 4)), {})
        assert value == getattr(ccb, name), name
    # both sit in reserved bytes of stripe lines, clear of word 0 and the tree's top
    for word in (ccb.CCB_XCD_COUNT_WORD, ccb.CCB_XCD_FLAG_WORD):
        assert word % 32 >= 1 and word % 32 + 8 <= 32 and word + 8 <= ccb.CCB_STRIPES * 32
        assert not (word <= ccb.CCB_TREE_TOP_WORD < word + 8)
    assert ccb.ccb_syncall_workspace_bytes(1) == (ccb.CCB_STRIPES + 1) * 128
    assert ccb.ccb_syncall_workspace_bytes(3) == (3 * ccb.CCB_STRIPES + 1) * 128
    # 2^26 elements in chunks of 1024, 1024 workgroups: 64 chunks each
    assert ccb.ccb_stencil_halo_bytes(1 << 26, 256, 1024) == 2 * 1024 * 64 * 2 * 4
    assert ccb.ccb_stencil_halo_bytes((1 << 20) + 1, 256, 1024) == 2 * 1024 * 2 * 2 * 4
    assert ccb.ccb_stencil_halo_bytes(0, 256, 4) == 0


def test_validation_before_device_work(ccb):
    # CntNotify §4.1: flag must be 0; a null out-pointer is rejected
    assert ccb.ccb_cnt_notify_create(1)[0] == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_cnt_notify_create(0, null_out=True)[0] == ccb.CCB_ERR_NULL_POINTER
    # §6.1: an unknown handle is an error, not a crash
    for bogus in (None, 1, 0x12345, (5 << 20) | 3):
        assert ccb.ccb_cnt_notify_record(bogus, None, ccb.record_info(1, 1)) == ccb.CCB_ERR_INVALID_HANDLE
        assert ccb.ccb_cnt_notify_wait(bogus, None, ccb.wait_info(3, 1, 1)) == ccb.CCB_ERR_INVALID_HANDLE
        assert ccb.ccb_cnt_notify_reset(bogus) == ccb.CCB_ERR_INVALID_HANDLE
        assert ccb.ccb_cnt_notify_get_id(bogus)[0] == ccb.CCB_ERR_INVALID_HANDLE
        assert ccb.ccb_cnt_notify_destroy(bogus) == ccb.CCB_ERR_INVALID_HANDLE
    # barrier launchers: null and malformed arguments
    assert ccb.ccb_syncall_workspace_reset(None, 1) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_syncall_workspace_reset(128, 0) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_syncall_workspace_reset(64, 1) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_barrier_only(None, None, None, 1, 8, 64) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_run_barrier_only(128, None, None, -1, 8, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_barrier_only(128, None, None, 1, 8, 100) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_barrier_only(128, None, None, 1, 8, 64, 9) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_slot_rounds(128, None, 256, None, 0, 1, 8, 64) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_run_grouped_rounds(128, 256, 256, None, 0, 1, 7, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_stencil(None, 256, 10, 1, 128, 512, 64, 1, 64) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_run_stencil(4096, 4096, 10, 1, 128, 512, 64, 1, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_stencil(4100, 8192, 10, 1, 128, 512, 64, 1, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_stencil(4096, 8192, 10, 1, 128, None, 0, 1, 64) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_run_stencil(4096, 8192, 10, 1, 128, 512, 8, 1, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_stencil(4096, 8192, 10, 1, 128, 512, 64, 1, 64,
                               timeline=4100) == ccb.CCB_ERR_INVALID_VALUE  # misaligned stamps
    # a mode is one layout (0 striped, 1 flat, 4 tree) ORed with one visibility
    # (0 order, 2 full, 8 per-XCD write-back)
    for bad in (5, 7, 10, 11, 13, 14, 15, 16, 18, -1):
        assert ccb.ccb_run_barrier_only(128, None, None, 1, 8, 64, mode=bad) == \
            ccb.CCB_ERR_INVALID_VALUE, bad
    # int32 stripes: (barriers + 1) * arrivals per stripe and barrier must stay below 2^31
    big = 2**31 // 4  # 256 members: 4 per stripe striped, 256 flat
    assert ccb.ccb_run_barrier_only(128, None, None, big, 256, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_barrier_only(128, None, None, 2**31 // 256, 256, 64,
                                    mode=ccb.CCB_BARRIER_FLAT) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_slot_rounds(128, 256, 256, None, 0, big, 256, 64) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_grouped_rounds(128, 256, 256, None, 0, 3 * (2**31 // 8), 512, 64) \
        == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_run_stencil(4096, 8192, 10, big + 1, 128, 512, 2**20, 256, 64) \
        == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_atomic_chain(None, 256, 1) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_bench_atomic_chain(128, 256, 0) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_copy(256, 512, 17) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_copy(None, 512, 16) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_bench_copy(264, 512, 16) == ccb.CCB_ERR_INVALID_VALUE  # misaligned dst
    # status: null, empty, oversized and misaligned workspaces are refused before any copy
    assert ccb.ccb_syncall_status(None, 1)[0] == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_syncall_status(128, 0)[0] == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_syncall_status(128, (1 << 20) + 1)[0] == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_syncall_status(64, 1)[0] == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_notify_pingpong(None, 256, 1, 1, 0, 256) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_bench_notify_pingpong(256, 256, 1, 1, 0, None) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_bench_notify_pingpong(256, 256, 0, 1, 0, 256) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_notify_pingpong(256, 256, 1, 0, 0, 256) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_notify_pingpong(256, 256, 1, 256, 0, 256) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_notify_pingpong(192, 256, 1, 1, 0, 256) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_notify_pingpong(256, 260, 1, 1, 0, 256) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_notify_pingpong(256, 256, 1, 1, 0, 258) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_hip_grid_sync(1, 8, 64, None) == ccb.CCB_ERR_NULL_POINTER
    assert ccb.ccb_bench_hip_grid_sync(0, 8, 64, 256) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_hip_grid_sync(1, 0, 64, 256) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_bench_hip_grid_sync(1, 8, 96, 256) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_cnt_notify_batch(None, None, -1, 1, None, None, 1) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_cnt_notify_batch(None, None, 0, 1, None, None, 1) == ccb.CCB_OK
    # one workgroup of 256 threads per 256 counters, fewer than 2^31 workgroups
    assert ccb.ccb_cnt_notify_batch(256, 256, 2**39, 1, 256, 256, 1) == ccb.CCB_ERR_INVALID_VALUE
    assert ccb.ccb_cnt_notify_batch(None, None, 4, 1, 256, 256, 1) == ccb.CCB_ERR_NULL_POINTER
    # the error word takes an atomic store: it must be 4-B aligned
    assert ccb.ccb_cnt_notify_batch(256, 256, 4, 1, 256, 256, 1, err=258) == ccb.CCB_ERR_INVALID_VALUE


def test_device_api_test_kernels_built():
    """The device-API test kernels (tests/devapi) are built and export their
    launcher; the header they include is the public in-kernel API."""
    import ctypes
    lib_path = os.path.join(os.path.dirname(__file__), "devapi", "libccb_devapi.so")
    assert os.path.exists(lib_path), "run __graft_entry__.build()"
    lib = ctypes.CDLL(lib_path)
    assert hasattr(lib, "devapi_run")
    text = open(os.path.join(INCLUDE, "ccb_device.h")).read()
    for name in ("ccb_syncall_soft", "ccb_syncall_soft_ordered", "ccb_syncall_soft_flat",
                 "ccb_syncall_soft_bounded", "ccb_arrive", "ccb_await", "ccb_barrier"):
        assert name + "(" in text, name
    # the test launcher refuses unknown variants and missing buffers before any
    # HIP call (hipErrorInvalidValue = 1; a launch attempt would report more)
    V, I32, U32, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64
    lib.devapi_run.restype = ctypes.c_int
    lib.devapi_run.argtypes = [ctypes.c_int, V, V, V, V, U64, I32, I32, I32, I32, I32, U32, V]
    for variant in range(8):
        assert lib.devapi_run(variant, None, None, None, None, 0, 1, 1, 1, 64, 0, 0, None) == 1
