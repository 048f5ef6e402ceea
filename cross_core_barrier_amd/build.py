"""Build libccb.so in-tree with hipcc for gfx950.

    python -m cross_core_barrier_amd.build

The library is written next to this file; the Python binding loads it from
there and nowhere else.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libccb.so")
SOURCES = ["ccb_kernels.hip", "ccb_api.hip"]
HEADERS = [os.path.join(ROOT, "include", "ccb.h"), os.path.join(ROOT, "include", "ccb_device.h"),
           os.path.join(CSRC, "ccb_internal.h")]


# flags shared by every compile of the kernels (the library and its review)
CODE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17",
    # packed-FP32 instructions stay off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every atomic here is issued by one lane; the wave-level atomic
    # rewrite would only add a wait on the reply before the barrier's poll
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc_command(out: str, extra=()) -> list:
    return [
        "hipcc", *CODE_FLAGS, "-fPIC", "-shared", "-fvisibility=hidden", "-Wall",
        "-Wl,-soname,libccb.so",
        *extra,
        "-o", out,
        *[os.path.join(CSRC, s) for s in SOURCES],
    ]


def device_assembly(out: str) -> str:
    """Write the gfx950 assembly of the kernels, compiled exactly as in the
    library, to `out` (for reading the code the library runs)."""
    cmd = ["hipcc", *CODE_FLAGS, "-S", "--cuda-device-only", "-o", out,
           os.path.join(CSRC, "ccb_kernels.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc -S failed:\n" + res.stdout + res.stderr)
    return out


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
