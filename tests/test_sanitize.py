"""Host builds with AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The oracle (oracle/wall_oracle.c) with gcc, driven by
  tests/sanitize/oracle_checks.c over every oracle function (packed
  sequences, a window, the scalar gate, a sink, a row subset, argument
  errors); leak detection on.
* The C-ABI argument checks: wall_api.cpp compiled for the host alone with
  both sanitizers, linked with the library's other objects as built, and
  driven by tests/sanitize/abi_checks.c through every entry point's error
  paths (each call returns before its first HIP call).

A sanitizer report makes the program exit nonzero (-fno-sanitize-recover).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "channel_decay_softmax_amd", "csrc")
BUILD = os.path.join(ROOT, "channel_decay_softmax_amd", "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def run(cmd, env=None, timeout=300):
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert p.returncode == 0, f"{' '.join(cmd[:3])} ...: exit {p.returncode}\n{p.stdout[-3000:]}\n{p.stderr[-3000:]}"
    return p


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_checks")
    run(["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "wall_oracle.c"),
         os.path.join(HERE, "oracle_checks.c"), "-lm", "-o", exe])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    p = run([exe], env=env)
    assert "oracle checks passed" in p.stdout


def test_abi_checks_under_sanitizers(tmp_path):
    if not (os.path.exists(CLANGXX) and os.path.exists(CLANG)):
        pytest.skip("no ROCm clang")
    objs = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD) if f.endswith(".o") and f != "wall_api.o") \
        if os.path.isdir(BUILD) else []
    if not objs:
        from channel_decay_softmax_amd import build

        build.build()
        objs = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD) if f.endswith(".o") and f != "wall_api.o")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = str(tmp_path / "wall_api.o")
    # host code only: no device pass, so the sanitizers instrument host code alone
    run([CLANGXX, "-x", "hip", "--offload-host-only", "-std=c++17", "-fPIC",
         *[f for s in SAN for f in (["-Xarch_host", s] if s.startswith("-fsanitize") else [s])],
         *inc, "-c", os.path.join(CSRC, "wall_api.cpp"), "-o", api])
    drv = str(tmp_path / "abi_checks.o")
    run([CLANG, "-x", "c", "-std=c11", "-Wno-incompatible-pointer-types-discards-qualifiers",
         "-D__HIP_PLATFORM_AMD__", *SAN, *inc, "-I", os.path.join(ROCM, "include"),
         "-c", os.path.join(HERE, "abi_checks.c"), "-o", drv])
    exe = str(tmp_path / "abi_checks")
    run([CLANGXX, "-fsanitize=address,undefined", drv, api, *objs, "-L", os.path.join(ROCM, "lib"),
         "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    # the HIP runtime is loaded but never initialised by these calls; its own
    # allocations at exit are not this library's
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    p = run([exe], env=env)
    assert "all statuses as declared" in p.stdout
