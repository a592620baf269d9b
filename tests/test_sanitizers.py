"""AddressSanitizer / UndefinedBehaviorSanitizer runs of the host code (CPU only).

Two drivers, each built with gcc and with ROCm's clang, sanitizers on, and run:

- tests/sanitize/host_checks.cpp: the library's host half
  (speculative_sampling_verification_vocab_amd/csrc/sv_host.h, the same source
  libspecverify.so compiles): launch geometry, workspace layouts filled through
  exact-size heap buffers, and every entry point's argument checks at their
  limits (INT32_MAX sizes, NULL and misaligned pointers, host arrays of
  exactly K entries);
- tests/sanitize/oracle_checks.c: every function of oracle/oracle.c on small
  cases (both dtypes and modes, K = 0, V = 1, faults, -inf rows, probes,
  invalid cluster ids, the KV status cases) with exact-size buffers.

No GPU code is built here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
CLANG = "/opt/rocm/llvm/bin/clang"

COMPILERS = {"gcc": ("gcc", "g++"), "clang": (CLANG, CLANG + "++")}


def _available(cc):
    return shutil.which(cc) is not None or os.path.exists(cc)


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    return r.returncode, r.stdout, r.stderr


@pytest.mark.parametrize("compiler", sorted(COMPILERS))
def test_host_checks_under_sanitizers(compiler, tmp_path):
    cc, cxx = COMPILERS[compiler]
    if not _available(cxx):
        pytest.skip(f"{cxx} not installed")
    exe = str(tmp_path / "host_checks")
    subprocess.check_call([cxx, "-std=c++17", *SAN, "-Wall", "-o", exe,
                           os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp")])
    rc, out, err = _run(exe)
    assert rc == 0 and "host checks ok" in out, err[-4000:]
    assert "runtime error" not in err and "ERROR: AddressSanitizer" not in err, err[-4000:]


@pytest.mark.parametrize("compiler", sorted(COMPILERS))
def test_oracle_under_sanitizers(compiler, tmp_path):
    cc, cxx = COMPILERS[compiler]
    if not _available(cc):
        pytest.skip(f"{cc} not installed")
    exe = str(tmp_path / "oracle_checks")
    subprocess.check_call([cc, "-std=c99", *SAN, "-fno-fast-math", "-ffp-contract=off", "-Wall", "-o", exe,
                           os.path.join(ROOT, "oracle", "oracle.c"),
                           os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), "-lm"])
    rc, out, err = _run(exe)
    assert rc == 0 and "oracle checks ok" in out, err[-4000:]
    assert "runtime error" not in err and "ERROR: AddressSanitizer" not in err, err[-4000:]
