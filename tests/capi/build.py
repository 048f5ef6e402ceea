"""Builds tests/capi/capi_example.c into tests/capi/libccb_capi_example.so with
gcc as strict C11 (-Wall -Wextra -Werror), against include/ccb.h, libccb.so
and the HIP runtime.  Called by __graft_entry__.build(); the tests load it."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libccb_capi_example.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str) -> list:
    pkg = os.path.join(ROOT, "cross_core_barrier_amd")
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
            "-fvisibility=hidden", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
            "-o", out, os.path.join(HERE, "capi_example.c"),
            "-L", pkg, "-lccb", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            # found next to the package wherever the tree is copied
            "-Wl,-rpath,$ORIGIN/../../cross_core_barrier_amd",
            "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def build(verbose: bool = False, out: str = LIB) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("gcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
