"""A C99 program that uses the library through include/w4a16.h and the HIP
runtime's C API only (tests/c_abi/consumer.c), checked against the oracle.

CPU: the header compiles as C99 with warnings on, and the program links
against the built library, the oracle and the HIP runtime (every entry point
it calls resolves).  GPU: the program runs and its checks pass (device
packing bit-exact, dense M = 3 and M = 1 within the fp32 bound and bitwise
batch-invariant, LM-head argmax, routed product, a refused group size).
"""
import os
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "consumer.c")
LIBDIR = os.path.join(ROOT, "decode_w4a16_affine_amd")
ORADIR = os.path.join(ROOT, "oracle")
ROCM = "/opt/rocm"


def build(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("gcc or the HIP headers are not installed")
    for lib in (os.path.join(LIBDIR, "libw4a16.so"), os.path.join(ORADIR, "liboracle.so")):
        if not os.path.exists(lib):
            pytest.skip(f"{os.path.basename(lib)} is not built")
    exe = str(tmp_path / "consumer")
    cmd = [gcc, "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", exe,
           "-L", LIBDIR, "-lw4a16", "-L", ORADIR, "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{LIBDIR}:{ORADIR}:{os.path.join(ROCM, 'lib')}", "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_consumer_builds(tmp_path):
    build(tmp_path)


@pytest.mark.gpu
def test_c_consumer_runs(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = build(tmp_path)
    print("C consumer: pack, dense M=3/M=1, LM head, routed (N=300 K=512)", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout, r.stderr)
