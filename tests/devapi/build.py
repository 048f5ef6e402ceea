"""Builds the device-API test kernels (tests/devapi/devapi_kernels.hip) into
tests/devapi/libccb_devapi.so for gfx950, with the library's code-generation
flags.  Called by __graft_entry__.build(); the GPU tests only load it."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libccb_devapi.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-atomic-optimizer-strategy=None", "-Wall",
           "-I", os.path.join(ROOT, "include"), "-o", tmp,
           os.path.join(HERE, "devapi_kernels.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
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
