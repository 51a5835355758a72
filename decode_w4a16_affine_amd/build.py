"""Compile the HIP library in-tree: decode_w4a16_affine_amd/libw4a16.so (gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libw4a16.so")
SOURCES = [os.path.join(HERE, "csrc", "w4a16.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # the contract is explicit fma only, never reassociation or contraction
    "-ffp-contract=off", "-fno-fast-math",
    # no packed fp32 arithmetic (v_pk_fma_f32 and friends) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 16 kernel-argument dwords arrive in scalar registers at wave
    # launch (gfx950 argument preloading; older firmware runs a load prologue)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, extra=()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, "-o", LIB, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
