"""The C ABI from C: tests/capi/capi_example.c uses only include/ccb.h and the
HIP runtime's C API.  On the CPU it must compile as strict C11 (-Wall -Wextra
-Werror) and link against libccb.so; on the GPU, called in-process, it runs
the CntNotify producer/consumer pattern, a barrier launch, a batched-engine
launch and a stencil launch, and checks each result itself."""

import ctypes
import os
import runpy

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CAPI = os.path.join(ROOT, "tests", "capi")


def test_capi_example_compiles_as_c11(tmp_path):
    # libccb.so (soname libccb.so) loaded first satisfies the copy's dependency
    from cross_core_barrier_amd import ccb  # noqa: F401
    b = runpy.run_path(os.path.join(CAPI, "build.py"))
    out = b["build"](out=str(tmp_path / "libcapi.so"))
    lib = ctypes.CDLL(out)
    assert hasattr(lib, "ccb_capi_example")


@pytest.mark.gpu
def test_capi_example_runs():
    import torch  # noqa: F401  (the GPU is visible)
    print("[gpu case] C-ABI example: CntNotify record/wait, barrier 8 x 64 x 100, batch 1024 x 8, "
          "stencil 5000 x 3", flush=True)
    lib = ctypes.CDLL(os.path.join(CAPI, "libccb_capi_example.so"))
    lib.ccb_capi_example.restype = ctypes.c_int
    lib.ccb_capi_example.argtypes = [ctypes.c_char_p, ctypes.c_int]
    buf = ctypes.create_string_buffer(256)
    rc = lib.ccb_capi_example(buf, 256)
    assert rc == 0, buf.value.decode()
    assert "800 arrivals" in buf.value.decode() and "stencil fixed point" in buf.value.decode()
