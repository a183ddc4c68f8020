"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/native/host_sanitize_check.cpp drives every host entry point of spectra_host.cpp (layout
validation, sizes, the float64 calibration with its blocked products, eigen-solver, robust
pairs, value correction, and the error paths) on small seeded problems.  Built here with g++ and
-fsanitize=address,undefined (the HIP launchers are not part of it), any out-of-bounds access or
undefined behaviour aborts the run with a report.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "native", "host_sanitize_check.cpp")
HOST = os.path.join(ROOT, "spectral_transform_coding_amd", "csrc", "spectra_host.cpp")


def test_host_code_clean_under_address_and_undefined_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_sanitize_check")
    build = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
                            "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                            DRIVER, HOST, "-o", exe], capture_output=True, text=True)
    if build.returncode != 0 and "asan" in (build.stderr + build.stdout).lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-2000:]
    # verify_asan_link_order=0: the process may preload other libraries ahead of the runtime
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "OK: 0 failures" in run.stdout, report[-2000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
