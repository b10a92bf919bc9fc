"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host-side code (CPU only).

Two standalone drivers under tests/sanitize/ are built with gcc/g++ and
-fsanitize=address,undefined (nothing here is GPU code): one runs every oracle
entry point on small ragged inputs in every cache format and layout, the other
runs the C ABI's host-side argument validation (msa_api.hip compiled as plain
C++ against stub launchers that only count calls).  A sanitizer report or a
wrong status fails the test.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None):
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=600, env=env)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p.stdout


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return tmp_path_factory.mktemp("sanitize")


def test_oracle_under_asan_ubsan(outdir):
    exe = str(outdir / "oracle_driver")
    _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *FLAGS, os.path.join(SAN, "oracle_driver.c"), "-o", exe,
          "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1")
    assert "oracle sanitizer run ok" in _run([exe], env)


def test_abi_validation_under_asan_ubsan(outdir):
    exe = str(outdir / "abi_driver")
    _run(["g++", "-std=c++17", "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "block_sparse_attention_index_amd", "csrc"),
          *FLAGS, os.path.join(SAN, "abi_driver.cpp"), "-o", exe])
    assert "abi sanitizer run ok" in _run([exe], dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
