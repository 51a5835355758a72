"""The CPU-side C code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two instrumented builds, each driven by an existing CPU test module in a
child process that preloads clang's sanitizer runtime:
  * the oracle (oracle/oracle.c), built with clang, under the oracle pins
    (tests/test_oracle_pins.py) through W4A16_ORACLE_LIB;
  * the C-ABI translation unit of the library (csrc/w4a16.hip: argument
    validation, status strings, schedule names, workspace sizes), host code
    instrumented (the device code of that unit is built as usual), with the
    per-row-count kernels replaced by stand-ins (tests/sanitize/host_stubs.hip),
    under the host ABI tests (tests/test_abi_host.py) through W4A16_LIB.
A deliberate heap overflow built with the same flags must abort, which shows
the runtime is live.  Any sanitizer report aborts the child (halt_on_error,
no recovery), so the test fails.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime():
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts or not os.path.exists(CLANG):
        pytest.skip("clang's sanitizer runtime is not installed")
    return rts[-1]


def _env(rt, **extra):
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **extra)
    env.pop("PYTEST_ADDOPTS", None)
    return env


def _run(cmd, env, timeout=300):
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def test_sanitizer_runtime_catches_a_planted_overflow(tmp_path):
    rt = _runtime()
    exe = str(tmp_path / "oob")
    subprocess.run([CLANG, *SAN, "-shared-libasan", "-o", exe, os.path.join(ROOT, "tests", "sanitize", "oob.c")],
                   check=True)
    rc, out = _run([exe], _env(rt))
    assert rc != 0 and "heap-buffer-overflow" in out, out[-2000:]


def test_oracle_pins_under_asan_ubsan(tmp_path):
    rt = _runtime()
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run([CLANG, "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", *SAN, "-o", lib,
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    env = _env(rt, W4A16_ORACLE_LIB=lib)
    probe = ("import oracle; oracle.lib(); m = open('/proc/self/maps').read(); "
             f"assert {lib!r} in m and 'libclang_rt.asan' in m, 'instrumented oracle not loaded'")
    rc, out = _run([sys.executable, "-c", probe], env)
    assert rc == 0, out[-3000:]
    rc, out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                    os.path.join(ROOT, "tests", "test_oracle_pins.py")], env)
    assert rc == 0, out[-3000:]


def test_abi_validation_under_asan_ubsan(tmp_path):
    rt = _runtime()
    lib = str(tmp_path / "libw4a16_san.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-x", "hip", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "decode_w4a16_affine_amd", "csrc"),
           "-o", lib, os.path.join(ROOT, "decode_w4a16_affine_amd", "csrc", "w4a16.hip"),
           os.path.join(ROOT, "tests", "sanitize", "host_stubs.hip")]
    for f in SAN:   # host code only
        cmd[1:1] = ["-Xarch_host", f]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = _env(rt, W4A16_LIB=lib)
    probe = ("import decode_w4a16_affine_amd as w4; w4.lib(); m = open('/proc/self/maps').read(); "
             f"assert {lib!r} in m and 'libclang_rt.asan' in m, 'instrumented library not loaded'")
    rc, out = _run([sys.executable, "-c", probe], env)
    assert rc == 0, out[-3000:]
    rc, out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                    os.path.join(ROOT, "tests", "test_abi_host.py")], env)
    assert rc == 0, out[-3000:]
