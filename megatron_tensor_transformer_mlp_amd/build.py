"""Build libmshard.so (HIP, gfx950 only) in-tree with hipcc.

    python -m megatron_tensor_transformer_mlp_amd.build

The library is written next to this file so that it travels with the source
tree; nothing is installed.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmshard.so")
SOURCES = ["kernels.hip", "attention.hip", "fingerprint.hip", "abi.cpp"]
HEADERS = ["gemm_core.hpp", "epilogues.hpp", "launch.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wno-inline-asm",  # the direct-to-LDS asm declares its M0 clobber on purpose
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]

# Per-source additions.  The attention kernels read every score and update
# every O accumulator with VALU instructions between their MFMAs; with the
# MFMA destinations in VGPRs they skip the AGPR-to-VGPR copies and need fewer
# registers in all (three waves per SIMD for head size 64 instead of two).
SOURCE_FLAGS = {
    "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l
                    and "argument unused during compilation: '--hip-link'" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build_library(verbose: bool = True, jobs: int = 2) -> str:
    """Compile every source for gfx950 and link libmshard.so; returns its path."""
    with tempfile.TemporaryDirectory(prefix="mshard_build_") as tmp:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            cmd = [HIPCC, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        for cmd, p in procs:
            out, _ = p.communicate()
            out = "\n".join(l for l in out.splitlines()
                            if "packed-fp32-ops' is not a recognized feature" not in l)
            if p.returncode != 0:
                raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
            if verbose and out.strip():
                print(out, flush=True)
        tmp_lib = LIB_PATH + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose="-q" not in sys.argv)
    print(LIB_PATH)
