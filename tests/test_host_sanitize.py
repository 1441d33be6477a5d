"""Host half of the library under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner, the tail-balancing model and the C ABI shim are built with g++
(-fsanitize=address,undefined, no recovery) against host stubs of the four
HIP runtime calls and the kernel launchers (tests/c/host_stubs.cpp), then
driven (tests/c/host_driver.cpp) over 1800 plans -- every policy, schedule,
history cap, conditioning and query length of a B <= 12, K <= 6 grid, plus
the 832x480 seven-chunk and long-video plans -- through every entry point,
with valid and invalid arguments, and with the memoised tail-balancing
choice queried from several threads at once.  Any sanitizer report or
failed check fails the test.  No GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_causal_attention_wave_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_asan")
    srcs = [os.path.join(CSRC, f) for f in ("planner.cpp", "balance.cpp", "abi.cpp")]
    srcs += [os.path.join(ROOT, "tests", "c", f) for f in ("host_stubs.cpp", "host_driver.cpp")]
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", exe, "-pthread"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-6000:])
    assert "ERROR: AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr
    plans, launches = int(run.stdout.split()[1]), int(run.stdout.split()[3])
    assert plans == 1802 and launches > 200000
