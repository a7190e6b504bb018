"""The CPU-side code under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (oracle/qmv_oracle.c, plain C) is built with gcc and both
  sanitizers and driven through every entry point, every bit width and
  group size and its error returns (tests/sanitize/oracle_driver.c).
* The library's host code (argument validation, workspace sizing, the
  thread-local error message) is built with the sanitizers on the host side
  only and driven with arguments it must refuse before any HIP call
  (tests/sanitize/abi_driver.cpp); no GPU is used.  That build takes about
  1.5 minutes and is cached under _build/sanitize, keyed by the sources.

Both runs abort on the first report (-fno-sanitize-recover=all)."""
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "bit_affine_quantized_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/bin/amdclang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    rc, log = _run(["gcc", "-std=c99", "-O1", "-ffp-contract=off", *SAN,
                    os.path.join(ROOT, "oracle", "qmv_oracle.c"),
                    os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe])
    assert rc == 0 and log.strip().endswith("ok"), log


def _sanitized_library():
    """libqmv with AddressSanitizer/UBSan on its host code, rebuilt when the
    sources change."""
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".h") or f == "qmv_api.hip")
    srcs.append(os.path.join(ROOT, "include", "qmv.h"))
    h = hashlib.sha256()
    for p in srcs:
        with open(p, "rb") as f:
            h.update(f.read())
    lib = os.path.join(OUT, "libqmv_hostsan_%s.so" % h.hexdigest()[:12])
    if not os.path.exists(lib):
        os.makedirs(OUT, exist_ok=True)
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "-std=c++17", "-O1", "-fPIC", "-shared", "--offload-arch=gfx950",
               "-Xarch_host", "-fsanitize=address,undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-g",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               os.path.join(CSRC, "qmv_api.hip"), "-o", tmp]
        rc, log = _run(cmd, timeout=900)
        assert rc == 0, log
        os.replace(tmp, lib)
    return lib


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not installed")
def test_abi_host_validation_under_asan_ubsan():
    lib = _sanitized_library()
    exe = os.path.join(OUT, "abi_driver")
    rc, log = _run([CLANG, "-std=c++17", *SAN, "-pthread", "-I", os.path.join(ROOT, "include"),
                    os.path.join(HERE, "abi_driver.cpp"), lib,
                    "-Wl,-rpath," + os.path.dirname(lib), "-o", exe])
    assert rc == 0, log
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0"   # the HIP runtime keeps process-lifetime allocations
    rc, log = _run([exe], env=env)
    assert rc == 0 and log.strip().endswith("ok"), log
