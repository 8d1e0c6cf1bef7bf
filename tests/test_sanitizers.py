"""The CPU-side C++ under the address and undefined-behaviour sanitizers.

- The library's host-only checks (csrc/hga_validate.cpp, and the workspace
  layouts and staging checks of csrc/hga_layout.h) are built with g++ and the
  sanitizers together with tests/sanitize_validate.cpp, which drives them over
  200,000 seeded shapes and argument sets (ordinary, boundary and extreme
  values) and checks every accepted one against the limits include/hga.h
  states, with the workspace sizes recomputed in 128-bit arithmetic.
- The oracle is built with the sanitizers and the whole CPU test suite runs
  against it, with the sanitizer runtimes preloaded into the interpreter.
Any sanitizer report aborts the run (halt_on_error), so a clean exit means no
out-of-bounds access, use after free, signed overflow or other undefined
behaviour on these paths.  Host only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _runtime(name):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not available")
    return path


def _env(tmp_path, oracle_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HGA_ORACLE_LIB"] = oracle_lib
    return env


def test_host_checks_under_sanitizers(tmp_path):
    _runtime("libasan.so")
    exe = str(tmp_path / "sanitize_validate")
    cmd = ["g++", "-std=c++17", "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "hierarchical_routed_sparse_amd", "csrc"),
           os.path.join(ROOT, "hierarchical_routed_sparse_amd", "csrc", "hga_validate.cpp"),
           os.path.join(ROOT, "tests", "sanitize_validate.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 violations" in r.stdout


def test_cpu_suite_against_sanitized_oracle(tmp_path):
    import oracle
    lib = oracle.build(force=True, out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    env = _env(tmp_path, lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m",
                        "not gpu", "-q", "-p", "no:cacheprovider", "-k", "not sanitizers"],
                       capture_output=True, text=True, timeout=900, env=env, cwd=ROOT)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail
