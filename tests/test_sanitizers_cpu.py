"""Host sanitizer builds (no GPU): the CPU oracle and the C ABI's host code (argument checks,
workspace sizes and launch geometry) run under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle is compiled with gcc; the ABI layer (abi.cpp) with hipcc, sanitizers on the host side
only, and linked with the library's ordinary kernel objects.  Each driver aborts on the first
out-of-bounds access or undefined operation and prints OK otherwise."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
OUT = os.path.join(ROOT, "_build", "san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_san")
    run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "oracle"), "-o", exe,
         os.path.join(NATIVE, "oracle_san_main.c"), os.path.join(ROOT, "oracle", "hs_oracle.c"),
         "-lm"])
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stderr[-3000:]


def test_abi_host_code_under_asan_ubsan():
    from oracle_top_kv_amd import build as hip_build
    kern = [os.path.join(hip_build.BUILD, os.path.basename(s) + ".o") for s in hip_build.sources()
            if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kern):
        hip_build.build()
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + hip_build.CSRC]
    abi_o, main_o, exe = (os.path.join(OUT, n) for n in ("abi.o", "main.o", "abi_san"))
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC"] + san + inc +
        ["-c", os.path.join(hip_build.CSRC, "abi.cpp"), "-o", abi_o])
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17"] + san + inc +
        ["-c", os.path.join(NATIVE, "abi_san_main.cpp"), "-o", main_o])
    run([HIPCC, "--offload-arch=gfx950"] + san[:4] + ["-o", exe, main_o, abi_o] + kern)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), (r.stdout[-2000:],
                                                                  r.stderr[-3000:])
