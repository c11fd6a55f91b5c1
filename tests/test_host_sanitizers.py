"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

tests/host_check.cpp drives every planner, workspace-size function and
argument check of the C ABI with valid, edge and invalid inputs (random
length arrays, extreme sizes up to INT_MAX, bad strides and pointers, unit
buffers of exactly max_units entries). It is linked against objects of the
library whose host code is instrumented (-fsanitize applies to the host side
only; the device code is compiled as usual and never runs here), so an
out-of-bounds access, a signed overflow or an invalid shift in host code fails
the test. The instrumented binary is rebuilt (about a minute and a half) only
when a source changes.
"""
import hashlib
import os
import subprocess

import pytest

from flashattention_attention_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_attention_amd", "csrc")
OUT = os.path.join(ROOT, "flashattention_attention_amd", "_build", "sanitize")
DRIVER = os.path.join(ROOT, "tests", "host_check.cpp")
HEADER = os.path.join(ROOT, "include", "fa.h")
# each sanitizer flag applies to the host compilation only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _digest():
    h = hashlib.sha256()
    for p in [DRIVER, HEADER] + [os.path.join(CSRC, s) for s in sorted(os.listdir(CSRC))]:
        h.update(p.encode())
        h.update(open(p, "rb").read())
    h.update(" ".join(SAN).encode())
    return h.hexdigest()


def _build():
    exe = os.path.join(OUT, "host_check")
    stamp = os.path.join(OUT, "stamp")
    digest = _digest()
    if os.path.exists(exe) and os.path.exists(stamp) and open(stamp).read() == digest:
        return exe
    os.makedirs(OUT, exist_ok=True)
    hipcc = build.hipcc()
    base = ["--offload-arch=" + build.ARCH, "-O1", "-g", "-std=c++17", "-fPIC", "-I",
            os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-Wno-unused-command-line-argument"] + SAN
    jobs, objs = [], []
    for src in build.SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc] + base + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                           text=True)))
        objs.append(obj)
    drv = os.path.join(OUT, "host_check.o")
    jobs.append(("host_check.cpp", subprocess.Popen(
        [hipcc, "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include")] + SAN +
        ["-c", DRIVER, "-o", drv], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for src, p in jobs:
        out, err = p.communicate()
        assert p.returncode == 0, f"{src}:\n{err[-3000:]}"
    r = subprocess.run([hipcc] + SAN + [drv] + objs + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    with open(stamp, "w") as f:
        f.write(digest)
    return exe


def test_host_code_under_sanitizers():
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    exe = _build()
    # leak checking off: the HIP runtime keeps process-lifetime allocations
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "host checks passed" in r.stdout
