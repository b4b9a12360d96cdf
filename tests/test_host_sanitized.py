"""The host-side logic of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

host_checks.cpp holds everything of the library that runs on the host
without a GPU: configuration checks, page layout, the split plan, the
device-metadata contract check and the argument checks of every call.  It
builds without HIP, so g++ compiles it here with both sanitizers, together
with tests/host_checks_driver.cpp, which calls it with valid and invalid
arguments.  Any sanitizer report aborts the driver.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_absorb_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


def _build(tmp_path, flags):
    exe = str(tmp_path / "host_checks_driver")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-Wall", "-Wextra", "-Werror", *flags, f"-I{CSRC}",
           os.path.join(CSRC, "host_checks.cpp"), os.path.join(ROOT, "tests", "host_checks_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("sanitizers", ["address,undefined"])
def test_host_checks_under_sanitizers(tmp_path, sanitizers):
    exe = _build(tmp_path, [f"-fsanitize={sanitizers}", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "expectations met" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_host_checks_build_without_hip(tmp_path):
    """host_checks.cpp includes no HIP header: a plain g++ build (no ROCm
    include path) succeeds."""
    exe = _build(tmp_path, [])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
