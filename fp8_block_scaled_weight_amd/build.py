"""Build libfp8q.so in-tree: every HIP source for gfx950, linked into one shared library.

    python -m fp8_block_scaled_weight_amd.build

Objects go to ``_build/`` at the repository root; the library is written next to this
file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfp8q.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "quant.hip", "kv_quant.hip", "gemm.hip", "moe.hip", "attention.hip"]

# No fast-math: fp32 division and the residual FMA must be IEEE; denormals are kept.
# Packed fp32 instructions are disabled for all device code.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=fast",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
    # MFMA results feed VALU promotion FMAs: keep them in VGPRs (no AGPR round trip)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8q)")


def build(verbose: bool = False, save_temps: bool = False) -> str:
    """Compile every source (always, in parallel) and link libfp8q.so."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmd = [cc, *HIPFLAGS, "-c", path, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if save_temps:
            cmd.append("-save-temps=obj")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, cwd=BUILD, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{t}" for s, t in failed)
        raise RuntimeError("libfp8q build failed:\n" + msg)
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv)
    print(LIB)
