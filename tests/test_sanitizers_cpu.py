"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two libraries are rebuilt with -fsanitize=address,undefined into a temporary directory:
  * the oracle's fp64 attention (oracle/attention_ref.c), with gcc;
  * the C-ABI layer of libjoint_attn (csrc/joint_attn.cpp: validation, workspace and
    split arithmetic, stream tables, error reporting), with g++, linked against host-only
    stand-ins for the kernel launchers (tests/sanitize/launch_stubs.cpp) instead of the
    gfx950 kernels.
The CPU test suite (ABI validation and every oracle pin) then runs in a child process
against those builds, with the sanitizer runtime preloaded; any sanitizer report fails
the test.  With the stand-in launchers, valid calls also run their whole host path.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "joint_attention_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name: str) -> str | None:
    try:
        p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized_libs(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc/g++ not available")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime for gcc")
    d = tmp_path_factory.mktemp("sanitize")
    oracle_so = str(d / "liboracle_attention_san.so")
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                    "-ffp-contract=off"] + SAN +
                   [os.path.join(ROOT, "oracle", "attention_ref.c"), "-o", oracle_so, "-lm"],
                   check=True)
    abi_so = str(d / "libjoint_attn_san.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
                   + SAN + [os.path.join(CSRC, "joint_attn.cpp"),
                            os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
                            "-o", abi_so], check=True)
    return dict(asan=asan, oracle=oracle_so, abi=abi_so)


def test_cpu_suite_under_asan_and_ubsan(sanitized_libs):
    tests = sorted(f for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_") and f.endswith(".py")
                   and f != os.path.basename(__file__) and "gpu" not in f)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": sanitized_libs["asan"],
        # the interpreter and torch are not instrumented: no leak report at exit
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "ORACLE_ATTENTION_LIB": sanitized_libs["oracle"],
        "JOINT_ATTN_LIB": sanitized_libs["abi"],
        "JOINT_ATTN_STUB_LAUNCHERS": "1",
        "OMP_NUM_THREADS": "4",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"]
    cmd += [os.path.join("tests", f) for f in tests]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out
