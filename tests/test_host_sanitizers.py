"""libkvq2's host code (argument validation, decode planning, calibration)
built with the host address and undefined-behaviour sanitizers and run by a
C++ self-test (tests/host_sanitize/), with stub launchers in place of the HIP
kernels.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_decode_kvq_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "kvq2_host_selftest")
    srcs = [os.path.join(CSRC, "kvq2_host.cpp"), os.path.join(CSRC, "kvq2_calibrate.cpp"),
            os.path.join(CSRC, "kvq2_hqmq_host.cpp"),
            os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "host_selftest.cpp")]
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-pthread",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip("the host toolchain has no sanitizer runtime")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host selftest ok" in r.stdout
