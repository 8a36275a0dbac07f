"""The host-side builders under AddressSanitizer and UndefinedBehaviorSanitizer.

bsvf_host.cpp (block lists, granular block lists, the launch schedule, status
strings) is plain C++; it is built here with the host compiler, sanitizers on,
together with tests/host_sanitize.cpp, which feeds it seeded random frame
patterns (valid ones, invalid ones, capacities one short) and checks the
two-call protocol and the invariants of what comes back.  No device code is
compiled or run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_video_frame_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def host_sanitize_exe(tmp_path_factory):
    tmp_path = tmp_path_factory.mktemp("host_sanitize")
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "host_sanitize")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE, "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(ROOT, "tests", "host_sanitize.cpp"), os.path.join(CSRC, "bsvf_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower() and "cannot find" in (r.stderr or "").lower():
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.mark.parametrize("seed", [1, 2])
def test_builders_under_sanitizers(host_sanitize_exe, seed):
    exe = host_sanitize_exe
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "1500", str(seed)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) > 500   # most draws are valid patterns that were checked
