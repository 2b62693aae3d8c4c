"""Host code under sanitizers, on the CPU.

* The library's host sources (argument checks, storage geometry, launch
  planning) built with g++ and AddressSanitizer + UndefinedBehaviorSanitizer
  against stand-ins of the HIP calls and kernel launchers
  (``tests/host/abi_host_check.cpp``): every refusal leaves no side effect, a
  destroyed handle is refused and a second destroy is harmless, and the
  workspace ``ripe_workspace_bytes`` returns covers the partial states every
  launch of a call writes, over a sweep of shapes, row counts and forced
  launch choices (calls of more than 256 rows run a shorter last launch).
* The C oracle built with the same sanitizers, running the oracle pins in a
  child process that preloads the sanitizer runtime.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _gcc_file(name):
    return subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()


def test_library_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    csrc = os.path.join(ROOT, "self_speculative_verify_amd", "csrc")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", csrc,
                           os.path.join(ROOT, "tests", "host", "abi_host_check.cpp"),
                           os.path.join(csrc, "ripe_api.cpp"), os.path.join(csrc, "plan.cpp"),
                           "-o", exe])
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(res.stdout[-2000:], res.stderr[-4000:])
    assert res.returncode == 0, res.stderr[-4000:]
    assert res.stdout.strip().endswith("host checks passed")


def test_oracle_pins_under_sanitizers(tmp_path):
    import oracle
    asan = _gcc_file("libasan.so")
    if not os.path.isabs(asan):
        pytest.skip("no libasan for gcc")
    lib = oracle.build(force=True, out=str(tmp_path / "libripe_oracle_san.so"),
                       extra_flags=[*SAN, "-g"])
    env = dict(os.environ, RIPE_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1",
               OMP_NUM_THREADS="4")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle.py"),
           os.path.join(ROOT, "tests", "test_oracle_draft.py")]
    res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    print(res.stdout[-3000:], res.stderr[-3000:])
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
