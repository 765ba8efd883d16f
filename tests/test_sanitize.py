"""Host sanitizer tier: libpti's host code (packer, split/join, the argument
checks of every entry point) and the oracle, built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven by tests/sanitize/host_checks.cpp.

CPU only.  The HIP sources are compiled with the sanitizers on the host side
alone (each -fsanitize= directly after -Xarch_host); device code is built as
usual but never launched: every device call the driver makes fails its
argument checks before any HIP call.  The build is cached under
tests/sanitize/_build keyed by the sources' hash.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_twin_int8_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp")
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
BUILD = os.path.join(ROOT, "tests", "sanitize", "_build")
LIB_SOURCES = ["pti_host.cpp", "pti_gemv.hip", "pti_verify.hip", "pti_glue.hip", "pti_attn.hip", "pti_toy.cpp"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
CLANG_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _tool(name):
    p = os.path.join("/opt/rocm", "llvm" if name.startswith("clang") else "", "bin", name)
    return p if os.path.exists(p) else shutil.which(name)


def _hash():
    h = hashlib.sha256()
    files = [os.path.join(CSRC, s) for s in LIB_SOURCES] + [DRIVER, ORACLE_C]
    files += [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")]
    files.append(os.path.join(INCLUDE, "pti.h"))
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout + r.stderr)


def build_checks() -> str:
    exe = os.path.join(BUILD, "host_checks")
    stamp = os.path.join(BUILD, "host_checks.sha256")
    key = _hash()
    if os.path.exists(exe) and os.path.exists(stamp) and open(stamp).read() == key:
        return exe
    hipcc, clang, clangxx = _tool("hipcc"), _tool("clang"), _tool("clang++")
    if not (hipcc and clang and clangxx):
        pytest.skip("ROCm clang/hipcc not found")
    os.makedirs(BUILD, exist_ok=True)
    base = ["-O1", "-g", "-std=c++20", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
    hip = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    jobs = []
    for s in LIB_SOURCES:
        cmd = [hipcc] + (["-xhip"] if s.endswith(".cpp") else []) + hip + base + HOST_SAN
        jobs.append(cmd + ["-c", os.path.join(CSRC, s), "-o", os.path.join(BUILD, s + ".o")])
    jobs.append([clang, "-O1", "-g", "-std=c11", "-ffp-contract=off", *CLANG_SAN, "-c", ORACLE_C,
                 "-o", os.path.join(BUILD, "oracle.o")])
    jobs.append([clangxx, "-O1", "-g", "-std=c++20", f"-I{INCLUDE}", *CLANG_SAN, "-c", DRIVER,
                 "-o", os.path.join(BUILD, "host_checks.o")])
    with ThreadPoolExecutor(4) as ex:
        list(ex.map(_run, jobs))
    objs = [os.path.join(BUILD, s + ".o") for s in LIB_SOURCES] + [os.path.join(BUILD, "oracle.o"),
                                                                      os.path.join(BUILD, "host_checks.o")]
    _run([hipcc, "--offload-arch=gfx950", "-fsanitize=address,undefined", *objs, "-o", exe])
    with open(stamp, "w") as f:
        f.write(key)
    return exe


def test_host_code_under_asan_and_ubsan():
    exe = build_checks()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert r.returncode == 0 and "ALL OK" in r.stdout, out[-6000:]
