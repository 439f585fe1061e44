"""Build libgdn.so (HIP kernels for gfx950 + the C-ABI) in-tree with hipcc.

Usage: ``python -m linear_attention_recurrence_03_amd.build`` (or ``build()``
from the package entry file).  Always recompiles.
"""
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["gdn_api.cpp", "gdn_decode.hip", "gdn_chunk.hip", "gdn_chunk_head.hip",
           "gdn_chunk_lag.hip", "gdn_attn.hip", "gdn_noalloc.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
# Device code: gfx950 only; packed-fp32 instruction selection disabled.
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fgpu-flush-denormals-to-zero", "-munsafe-fp-atomics"]


# The decode and attention kernels have the hardware preload their leading kernel
# arguments (as many dwords as the user-SGPR budget leaves, 14 here) into scalar
# registers at wave launch (gfx950; the code keeps a fallback entry that loads
# them itself where the firmware does not).
_PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
PER_FILE = {"gdn_decode.hip": _PRELOAD, "gdn_attn.hip": _PRELOAD}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


TRACE_LIB = os.path.join(PKG, "libgdn_trace.so")


def build(verbose: bool = False, jobs: int = 4, trace: bool = False) -> str:
    """Compile libgdn.so; with ``trace`` the phase-timestamp variant libgdn_trace.so
    (-DGDN_PHASE_TRACE: the lag scan records per-wave phase timestamps)."""
    lib = TRACE_LIB if trace else LIB
    with tempfile.TemporaryDirectory(prefix="gdn_build_") as tmp:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            flags = COMMON + (DEVICE if src.endswith(".hip") else ["-D__HIP_PLATFORM_AMD__"])
            flags = flags + PER_FILE.get(src, [])
            if trace:
                flags = flags + ["-DGDN_PHASE_TRACE"]
            cmd = [HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd))
            objs.append(obj)
        bad = [p.wait() for p in procs]
        if any(bad):
            raise RuntimeError("hipcc failed (exit codes %s)" % bad)
        tmp_lib = lib + ".tmp"
        _run([HIPCC, "-shared", "--offload-arch=" + ARCH, "-fPIC", "-o", tmp_lib] + objs, verbose)
        os.replace(tmp_lib, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, trace="--trace" in sys.argv))
