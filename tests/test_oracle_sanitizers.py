"""The C oracle under AddressSanitizer + UndefinedBehaviorSanitizer, and its
host-thread epoch barrier under ThreadSanitizer (CPU only).

tests/sanitize/oracle_driver.c drives every oracle entry point on small inputs
and checks properties that hold by construction; here it is built with gcc and
each sanitizer, and must exit 0 with no sanitizer report."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "oracle", "ccb_oracle.c"), os.path.join(ROOT, "oracle", "host_barrier.c"),
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


def _build_and_run(flags, args):
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread", *flags, *SOURCES, "-o", exe]
        b = subprocess.run(cmd, capture_output=True, text=True)
        if b.returncode != 0 and "sanitize" in b.stderr and "cannot find" in b.stderr:
            pytest.skip("sanitizer runtime not installed")
        assert b.returncode == 0, b.stderr
        r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300)
        return r


def test_oracle_address_and_undefined_behaviour():
    r = _build_and_run(["-fsanitize=address,undefined", "-fno-sanitize-recover=all"], ["all"])
    assert r.returncode == 0, r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


def test_host_barrier_threads():
    r = _build_and_run(["-fsanitize=thread"], ["threads"])
    assert r.returncode == 0, r.stderr
    assert "ThreadSanitizer" not in r.stderr, r.stderr
