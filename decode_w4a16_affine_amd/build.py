"""Compile the HIP library in-tree: decode_w4a16_affine_amd/libw4a16.so (gfx950).

The decode kernels are instantiated once per activation-row count in separate
objects (csrc/inst.hip compiled with -DW4K_M=1..8), the prefill kernels and
the C ABI in two more, all compiled in parallel and linked into one library.
"""
import concurrent.futures as cf
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16.so")
PROBE_LIB = os.path.join(HERE, "libw4a16_probe.so")   # measurement kernels (benchmark only)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
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

# (object name, source, extra arguments)
UNITS = [(f"inst_m{m}", "inst.hip", [f"-DW4K_M={m}"]) for m in range(1, 9)] + [
    # matrix-core results in ordinary VGPRs: by default the compiler gives the
    # tiled prefill kernel's products to the accumulation registers and reads
    # every one back before its scaling fma (80 extra VALU per wave and step)
    ("prefill", "prefill.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("abi", "w4a16.hip", []),
]

_NOISE = "not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if _NOISE not in l)
    return r.returncode, err


def build_probe(verbose: bool = False) -> str:
    """libw4a16_probe.so: the streaming-read kernel the benchmark measures the read ceiling with."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", "-o", tmp, os.path.join(CSRC, "probe.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    rc, err = _run(cmd)
    if rc != 0:
        raise RuntimeError(f"hipcc failed ({rc}) on probe.hip:\n{err}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False, extra=(), out: str = LIB, jobs: int = None) -> str:
    jobs = jobs or max(1, min(len(UNITS), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="w4a16_build_") as tmp:
        cmds = []
        for name, src, defs in UNITS:
            obj = os.path.join(tmp, name + ".o")
            cmds.append((obj, [HIPCC, *FLAGS, *defs, *extra, "-c", "-o", obj, os.path.join(CSRC, src)]))
        if verbose:
            for _, c in cmds:
                print(" ".join(c), flush=True)
        with cf.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda oc: _run(oc[1]), cmds))
        for (obj, c), (rc, err) in zip(cmds, results):
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {os.path.basename(c[-1])} -> {os.path.basename(obj)}:\n{err}")
            if verbose and err.strip():
                print(err)
        tmp_lib = out + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib, *[o for o, _ in cmds]]
        if verbose:
            print(" ".join(link), flush=True)
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_probe(verbose=True)
