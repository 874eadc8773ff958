"""The attention, fingerprint and cross-entropy-gradient kernels' own sources, run
on the CPU (host emulation).

attention.hip and fingerprint.hip are compiled unmodified for the host with
tests/cpu_emu: each lane a fiber, one workgroup at a time, lanes meeting at
the workgroup barrier, and the three cross-lane operations the attention
kernels use emulated with their lane semantics:
  * v_mfma_f32_16x16x32_bf16 - lane l supplies row l%16, k = 8(l/16) .. +7 of
    the first operand and column l%16 of the second, and receives
    D[4(l/16) + r][l%16] (the layout the GEMM core relies on);
  * ds_read_b64_tr_b16 - within each 16-lane group, result lane i, element e
    is element i%4 of what source lane i/4 + 4e addressed (measured on the GPU);
  * the lane-pair swaps - both lanes of a pair receive (lower lane's value,
    upper lane's value).
The outputs are compared with the fp64 oracle (attention forward), torch's
fp64 autograd of scaled_dot_product_attention (its gradients) and the xxhash
library (fingerprints).  Arithmetic is fp32 with bf16 operands and outputs, so
the bar is the GPU bar: relative Frobenius error <= 1e-2; lse and fingerprints
much tighter.  This checks the kernel sources' indexing and control flow; it
does not replace running them on the GPU.

The cross-entropy backward's epilogue (EpiCEGrad in epilogues.hpp) is run the
same way over every tile of a ragged logit matrix, with tests/cpu_emu's
stand-in for the GEMM core (its accumulator lane layout, buffer resources that
read zero past their end and drop stores there).  epilogues.hpp is used as is,
except that its three inline-assembly statements are removed mechanically: an
LDS wait (every access is synchronous here) and two register reads of another
epilogue that is not compiled in.
"""
import re
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch
import xxhash

from megatron_tensor_transformer_mlp_amd import inputs
from oracle import attn
from tests.conftest import rel_fro

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "megatron_tensor_transformer_mlp_amd", "csrc")
EMU = os.path.join(ROOT, "tests", "cpu_emu")
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def drivers(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("clang++ not found")
    d = tmp_path_factory.mktemp("cpu_emu")
    for f in ("attention.hip", "fingerprint.hip", "launch.hpp"):
        shutil.copy(os.path.join(CSRC, f), d)            # the kernel sources, unmodified
    for f in ("epilogues.hpp", "attn_driver.cpp", "fp_driver.cpp"):
        shutil.copy(os.path.join(EMU, f), d)
    shutil.copytree(os.path.join(EMU, "hip"), os.path.join(d, "hip"))
    # the epilogue under its own name, beside the stand-in core, for the CE-gradient driver
    e = os.path.join(d, "ce")
    os.makedirs(e)
    src = open(os.path.join(CSRC, "epilogues.hpp")).read()
    src, n = re.subn(r"\basm\b(\s+volatile)?\s*\((?:[^()]|\([^()]*\))*\)\s*;", ";", src)
    assert n == 3 and "asm" not in re.sub(r"//[^\n]*", "", src)
    open(os.path.join(e, "epilogues.hpp"), "w").write(src)
    for f in ("gemm_core.hpp", "ce_grad_driver.cpp"):
        shutil.copy(os.path.join(EMU, f), e)
    shutil.copytree(os.path.join(EMU, "hip"), os.path.join(e, "hip"))
    out = {}
    for name, where in (("attn_driver", d), ("fp_driver", d), ("ce_grad_driver", e)):
        exe = os.path.join(where, name)
        subprocess.run([CLANG, "-std=c++20", "-O1", "-x", "c++", f"-I{where}", os.path.join(where, name + ".cpp"),
                        "-o", exe, "-lpthread"], check=True, capture_output=True)
        out[name] = exe
    return out, d


def _f64(u):
    return inputs.bf16_bits_to_f32(u).astype(np.float64)


@pytest.mark.parametrize("b,s,n,d,causal,rate", [(1, 64, 1, 16, True, 0), (2, 70, 2, 32, True, 0),
                                                 (1, 130, 1, 64, False, 0), (1, 96, 1, 96, True, 0),
                                                 (1, 64, 1, 128, False, 0), (3, 1, 2, 32, True, 0),
                                                 (1, 200, 1, 64, True, 0), (1, 200, 1, 64, True, 0.02),
                                                 (2, 200, 1, 32, False, 0.125)])
def test_attention_kernels_emulated(drivers, b, s, n, d, causal, rate):
    """rate > 0 scales key row t by 1 + rate * t, so later key steps raise the running max (and rescale O)
    while others stay within the forward's rescale slack."""
    exes, tmp = drivers
    rng = np.random.default_rng(b * 1000 + s * 10 + d)
    T, nd = b * s, n * d
    x = rng.standard_normal((T, 3 * nd)).astype(np.float32)
    x[:, nd:2 * nd] *= np.tile(1.0 + rate * np.arange(s), b)[:, None].astype(np.float32)
    qkv = inputs.round_to_bf16_bits(x)
    dout = inputs.round_to_bf16_bits(rng.standard_normal((T, nd)).astype(np.float32))
    case = os.path.join(tmp, f"attn_{b}_{s}_{n}_{d}_{int(causal)}_{rate}")
    os.makedirs(case, exist_ok=True)
    qkv.tofile(os.path.join(case, "qkv.bin"))
    dout.tofile(os.path.join(case, "dout.bin"))
    subprocess.run([exes["attn_driver"], str(b), str(s), str(n), str(d), str(int(causal)), case], check=True,
                   timeout=300)
    o = np.fromfile(os.path.join(case, "o.bin"), dtype=np.uint16).reshape(T, nd)
    lse = np.fromfile(os.path.join(case, "lse.bin"), dtype=np.float32).reshape(n, T)
    dqkv = np.fromfile(os.path.join(case, "dqkv.bin"), dtype=np.uint16).reshape(T, 3 * nd)
    Q, K, V = _f64(qkv[:, :nd]), _f64(qkv[:, nd:2 * nd]), _f64(qkv[:, 2 * nd:])
    want = attn.attention_core(Q, K, V, n, d, b, s, causal)
    qt, kt, vt = (torch.tensor(x.reshape(b, s, n, d).transpose(0, 2, 1, 3).copy(), requires_grad=True)
                  for x in (Q, K, V))
    ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    (ot * torch.tensor(_f64(dout).reshape(b, s, n, d).transpose(0, 2, 1, 3).copy())).sum().backward()

    def grad(t):
        return t.grad.numpy().transpose(0, 2, 1, 3).reshape(T, nd)

    g = _f64(dqkv)
    assert rel_fro(_f64(o), want["O"]) <= 1e-2
    assert rel_fro(lse, want["lse"]) <= 1e-5
    for got, t in ((g[:, :nd], qt), (g[:, nd:2 * nd], kt), (g[:, 2 * nd:], vt)):
        assert rel_fro(got, grad(t)) <= 1e-2


@pytest.mark.parametrize("nbytes,chunk", [(0, 64), (7, 8), (100, 32), (4099, 1024), (70000, 4096)])
def test_fingerprint_kernel_emulated(drivers, nbytes, chunk):
    exes, tmp = drivers
    data = np.random.default_rng(nbytes).integers(0, 256, size=nbytes, dtype=np.uint8).tobytes()
    src, dst = os.path.join(tmp, f"fp_{nbytes}.bin"), os.path.join(tmp, f"fp_{nbytes}.out")
    with open(src, "wb") as f:
        f.write(data)
    subprocess.run([exes["fp_driver"], src, str(nbytes), str(chunk), dst], check=True, timeout=300)
    words = np.fromfile(dst, dtype=np.uint64).tolist()
    parts = [data[k:k + chunk] for k in range(0, nbytes, chunk)] or [b""]
    assert words[1:] == [xxhash.xxh64(p).intdigest() for p in parts]
    assert words[0] == xxhash.xxh64(b"".join(w.to_bytes(8, "little") for w in words[1:])).intdigest()


def test_ce_gradient_epilogue_emulated(drivers):
    """dL = coef (exp(L - M) / S - one-hot) over a 300 x 520 logit block (2 x 3 tiles with
    ragged edges), targets on tile and shard edges and outside the shard, masked tokens."""
    exes, tmp = drivers
    M, N = 300, 520
    rng = np.random.default_rng(7)
    L = (rng.standard_normal((M, N)) * 3).astype(np.float32)
    tcol = rng.integers(0, N, size=M)
    tcol[:8] = [0, N - 1, 255, 256, 511, 512, -1, -1]          # tile and shard edges; not in this shard
    coef = rng.uniform(0.5, 1.5, size=M) / M
    coef[10:14] = 0.0                                          # masked tokens
    Ld = L.astype(np.float64)
    Mx = Ld.max(axis=1) + rng.uniform(0, 1, size=M)          # combined max over a larger vocabulary
    S = np.exp(Ld - Mx[:, None]).sum(axis=1) + rng.uniform(0, 5, size=M)
    rec = np.zeros((M, 4), dtype=np.float32)
    rec[:, 0] = (Mx * np.log2(np.e)).astype(np.float32)
    rec[:, 1] = (coef / S).astype(np.float32)
    rec[:, 2] = coef.astype(np.float32)
    rec = rec.view(np.uint32)
    rec[:, 3] = tcol.astype(np.int32).view(np.uint32)
    case = os.path.join(tmp, "ce_grad")
    os.makedirs(case, exist_ok=True)
    L.tofile(os.path.join(case, "logits.bin"))
    rec.tofile(os.path.join(case, "stats.bin"))
    subprocess.run([exes["ce_grad_driver"], str(M), str(N), case], check=True, timeout=300)
    dl_bits = np.fromfile(os.path.join(case, "dl.bin"), dtype=np.uint16).reshape(M, N)
    assert not (dl_bits == 0xFFFF).any()                       # every element written
    got = _f64(dl_bits)
    onehot = np.arange(N)[None, :] == tcol[:, None]
    want = coef[:, None] * (np.exp(Ld - Mx[:, None]) / S[:, None] - onehot)
    assert rel_fro(got, want) <= 1e-2
    np.testing.assert_allclose(got, want, rtol=2 ** -7, atol=1e-12)
    sel = (tcol >= 0) & (coef > 0)                             # the target column is a row's only negative entry
    assert (got[sel, tcol[sel]] < 0).all() and ((got < 0).sum(axis=1) == sel).all()
    assert not got[10:14].any()                                # masked tokens: exactly zero
