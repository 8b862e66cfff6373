"""Host-side memory and undefined-behaviour checks (CPU only): the fp64 oracle
and the host side of the C ABI (argument validation, workspace and scratch
sizes, kernel names), each built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through every entry point by a small
program under tests/pins/.  A sanitizer report aborts the program; the test
then fails with the report.

The ABI build instruments host code only (device code is compiled as usual)
and links the kernel objects that build.py left in the package's _build
directory; nothing is launched, so no GPU is needed.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "pins")
ROCM = "/opt/rocm"
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
BUILD = os.path.join(ROOT, "exact_attention_79_amd", "_build")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc is not installed")
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         os.path.join(PINS, "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "attn_oracle.c"),
         "-lm", "-o", exe])
    out = run([exe], env=SAN_ENV)
    assert "oracle under sanitizers: ok" in out


def test_abi_layer_under_asan_ubsan(tmp_path):
    objs = [os.path.join(BUILD, f"{n}.o") for n in ("attn_fwd", "attn_bwd", "attn_decode")]
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX) and all(map(os.path.exists, objs))):
        pytest.skip("hipcc, ROCm's clang++ or the built kernel objects are missing")
    api = str(tmp_path / "attn_api_san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I" + os.path.join(ROOT, "include"), "-c",
         os.path.join(ROOT, "exact_attention_79_amd", "csrc", "attn_api.hip"), "-o", api])
    exe = str(tmp_path / "abi_san")
    run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"),
         os.path.join(PINS, "abi_sanitize_main.cpp"), api, *objs,
         "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
         "-o", exe])
    # The HIP runtime itself is not instrumented and keeps allocations for
    # the process's lifetime; leaks are checked in the oracle test only.
    env = dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    out = run([exe], env=env)
    assert "ABI layer under sanitizers: ok" in out
