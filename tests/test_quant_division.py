"""The encode kernel's division-free quantiser step equals IEEE float32 division.

The matrix-core encode kernel replaces c / s by a reciprocal per group and one fused
multiply-add correction per element (Markstein's step).  The codes then stay bit-identical to
the quantiser's definition only if that sequence returns the correctly rounded quotient for every
float32 c and every fp16 scale s.  This test compiles a small C program (plain host float
arithmetic, nothing shared with the HIP code) and checks every float32 significand of c against a
spread of fp16 significands of s, the all-ones one included.  The full sweep over all 1024
significands (8.6e9 pairs) ran clean when the kernel adopted the sequence; set
SPECTRA_DIV_EXHAUSTIVE=1 to repeat it here (about 10 s on 8 cores).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "quant_division_check.c")


def _cpu_has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read() + " "
    except OSError:
        return False


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("divchk") / "quant_division_check")
    flags = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]
    if _cpu_has_fma():
        flags.append("-mfma")          # hardware fused multiply-add; fmaf is exact either way
    subprocess.run(["gcc", *flags, SRC, "-o", exe, "-lm"], check=True)
    return exe


def _run(exe, first, last, stride):
    p = subprocess.run([exe, str(first), str(last), str(stride)], capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout.strip()


def test_markstein_step_matches_ieee_division(checker):
    if os.environ.get("SPECTRA_DIV_EXHAUSTIVE") == "1":
        rc, out = _run(checker, 0, 1024, 1)
        assert rc == 0, out
        assert out == f"checked {1024 << 23} mismatches 0"
        return
    # every 37th significand (28 of them, spread over the binade) plus the two ends
    for first, last, stride in ((0, 1024, 37), (1023, 1024, 1), (1, 2, 1)):
        rc, out = _run(checker, first, last, stride)
        assert rc == 0, out


def test_checker_detects_an_uncorrected_quotient(tmp_path):
    """The same program without the correction step must report mismatches (the check has teeth)."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(SRC).read().replace("fmaf(fmaf(-q0, s, c), r, q0)", "q0")
    assert "= q0;" in src
    p = tmp_path / "nocorr.c"
    p.write_text(src)
    exe = str(tmp_path / "nocorr")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", str(p), "-o", exe, "-lm"], check=True)
    rc, out = _run(exe, 3, 4, 1)
    assert rc == 1 and "mismatches 0" not in out, out
