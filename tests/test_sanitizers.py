"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

- The C ABI's argument checks (sas_api.cpp), linked against stand-in kernel
  launchers and HIP runtime calls: every entry point with good and bad
  arguments, host arrays at exactly their documented sizes
  (tests/sanitizers/api_harness.cpp).
- The oracle (oracle/sas_oracle.c): every entry point on small ragged
  problems, every gate mode, with and without row / key-block masks
  (tests/sanitizers/oracle_harness.c).
Both are built here with the host compilers only (no device code) and must
run clean: a sanitizer report aborts the program.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")
def test_abi_checks_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "api_harness")
    run([CLANG, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-I" + os.path.join(ROOT, "include"),
         "-I" + os.path.join(ROOT, "trainable_block_sparse_gate_amd", "csrc"),
         os.path.join(ROOT, "trainable_block_sparse_gate_amd", "csrc", "sas_api.cpp"),
         os.path.join(ROOT, "tests", "sanitizers", "api_harness.cpp"), "-o", exe])
    r = run([exe])
    assert "0 failures" in r.stdout, r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_harness")
    run(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off",
         os.path.join(ROOT, "oracle", "sas_oracle.c"),
         os.path.join(ROOT, "tests", "sanitizers", "oracle_harness.c"), "-o", exe, "-lm"])
    r = run([exe], env=dict(os.environ, OMP_NUM_THREADS="4"))
    assert "0 failures" in r.stdout, r.stdout
