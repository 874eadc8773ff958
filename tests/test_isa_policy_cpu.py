"""Instruction-level checks of the built library's gfx950 code (CPU only).

Disassembles the device code object embedded in libmshard.so and checks that
no kernel contains:
  * a write through the scalar data cache (scalar memory stores and atomics,
    the scalar cache's write-back and discard);
  * a packed-fp32 VALU instruction (the build disables them);
  * an atomic of any kind (global, buffer, flat or LDS), which backs the
    library's bitwise-determinism guarantee at the instruction level.
This file names those instructions, so it is a host-side checker only.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

LLVM = "/opt/rocm/llvm/bin"
TOOLS = ("llvm-readelf", "llvm-objdump", "clang-offload-bundler")


@pytest.fixture(scope="module")
def mnemonics():
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in TOOLS):
        pytest.skip("ROCm LLVM tools not found")
    from megatron_tensor_transformer_mlp_amd import build
    so = build.LIB_PATH
    if not os.path.exists(so):
        build.build_library(verbose=False)
    sec = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "-SW", so], capture_output=True, text=True,
                         check=True).stdout
    line = next(l for l in sec.splitlines() if ".hip_fatbin" in l)
    fields = line.split("]", 1)[1].split()
    off, size = int(fields[3], 16), int(fields[4], 16)
    tmp = tempfile.mkdtemp(prefix="mshard_isa_")
    try:
        with open(so, "rb") as f:
            f.seek(off)
            blob = f.read(size)
        fb, co = os.path.join(tmp, "fatbin"), os.path.join(tmp, "gfx950.co")
        with open(fb, "wb") as f:
            f.write(blob)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={fb}", f"--output={co}"], check=True)
        text = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--no-show-raw-insn", co],
                              capture_output=True, text=True, check=True).stdout
    finally:
        shutil.rmtree(tmp)
    ops = [m.group(1) for m in re.finditer(r"^\s+([a-z_][a-z0-9_]*)\b", text, flags=re.M)]
    assert len(ops) > 10000, "disassembly looks empty"
    return set(ops)


def test_kernels_are_present(mnemonics):
    assert any(op.startswith("v_mfma_f32_16x16x32") for op in mnemonics)
    assert "ds_read_b64_tr_b16" in mnemonics


def test_no_scalar_cache_writes(mnemonics):
    bad = sorted(op for op in mnemonics
                 if re.match(r"s_(buffer_|scratch_)?(store|atomic)", op) or re.match(r"s_dcache_(wb|discard)", op))
    assert not bad, bad


def test_no_packed_fp32_valu(mnemonics):
    bad = sorted(op for op in mnemonics if re.match(r"v_pk_(add|mul|fma)_f32", op))
    assert not bad, bad


def test_no_atomics(mnemonics):
    bad = sorted(op for op in mnemonics
                 if "atomic" in op or re.match(r"ds_(add|sub|inc|dec|min|max|and|or|xor|cmpst|wrap)", op))
    assert not bad, bad
