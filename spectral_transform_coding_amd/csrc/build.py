"""Builds libspectra.so in-tree: host C++ with g++ (OpenMP), HIP kernels with hipcc for gfx950.

    python spectral_transform_coding_amd/csrc/build.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspectra.so")

HOST_SOURCES = ["spectra_host.cpp"]
HIP_SOURCES = ["spectra_encode.hip", "spectra_decode.hip", "spectra_literal.hip"]
ARCH = os.environ.get("SPECTRA_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # packed fp32 arithmetic is left to no one: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wno-unused-result",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


# Device headers embedded (as one string) for run-time specialisation of the decode kernel.
JIT_HEADERS = [os.path.join(ROOT, "include", "spectra.h"), os.path.join(HERE, "spectra_internal.h"),
               os.path.join(HERE, "spectra_device.h"), os.path.join(HERE, "spectra_decode_mfma.h")]


def write_jit_source() -> str:
    """_build/spectra_jit_source.inc: the headers with their #include / #pragma once lines removed
    (hiprtc compiles one self-contained translation unit), as a raw string literal."""
    import re
    parts = ["#include <cstdint>\n"]
    for h in JIT_HEADERS:
        t = open(h).read()
        t = re.sub(r'^\s*#\s*(include\s*[<"][^>"]+[>"]|pragma\s+once)\s*$', "", t, flags=re.M)
        parts.append(f"// ---- {os.path.basename(h)}\n" + t)
    text = "\n".join(parts)
    assert ')spectra_jit"' not in text
    out = os.path.join(BUILD, "spectra_jit_source.inc")
    body = 'static const char kJitSource[] = R"spectra_jit(' + text + ')spectra_jit";\n'
    if not os.path.exists(out) or open(out).read() != body:
        open(out, "w").write(body)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    write_jit_source()
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", "-O3", "-fPIC", "-std=c++17", "-fopenmp", "-Wall", "-c",
              os.path.join(HERE, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        path = os.path.join(HERE, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, src + ".o")
        out = _run([HIPCC] + HIP_FLAGS + [f"-I{BUILD}", "-c", path, "-o", obj])
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    gomp = subprocess.run(["g++", "-print-file-name=libgomp.so"], capture_output=True,
                          text=True).stdout.strip()
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs +
         [f"-L{os.path.dirname(gomp)}", "-lgomp", "-Wl,-rpath," + os.path.dirname(gomp),
          "-L/opt/rocm/lib", "-lhiprtc", "-Wl,-rpath,/opt/rocm/lib"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
