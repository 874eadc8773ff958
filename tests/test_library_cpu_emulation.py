"""The whole library's launch sequences run on the CPU, against the fp64 oracle.

tests/cpu_emu/prep.py copies every kernel source of the library (the GEMM core
and its epilogues included), replacing each inline-assembly statement by its
emulated meaning; tests/cpu_emu/hip/hip_runtime.h runs each workgroup's lanes
as fibers that meet at barriers, with emulated MFMA, direct-to-LDS loads,
transposing LDS reads, buffer resources (out-of-range loads read zero, stores
are dropped) and lane exchanges.  tests/cpu_emu/lib_driver.cpp calls the library's own launch
functions (kernels.hip, attention.hip): the same launch plans, workspace
layouts, paired and split-K launches, grids and kernel arguments as on the GPU.

What this shows: indexing, tiling, masking of ragged edges, the K tail, split-K
slices and their fixed-order reduction, paired launches, workspace offsets and
every epilogue compute the definitions the oracle writes out.  What it does not
show: anything about timing on the GPU (the direct-to-LDS loads land at once
here, where the hardware needs the kernels' own waits and barriers), nor the
hardware's exp2 and reciprocal rounding.  Outputs and workspaces start as NaN,
so an element left unwritten fails.  Tolerances are those of the GPU parity
tests: relative Frobenius 1e-2 for bf16-input GEMM outputs and gradients, 1e-4
for the CE partials, the per-token loss and its mean.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_mlp_amd import inputs
from oracle import attn
from tests.conftest import rel_fro

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "megatron_tensor_transformer_mlp_amd", "csrc")
EMU = os.path.join(ROOT, "tests", "cpu_emu")
CLANG = "/opt/rocm/llvm/bin/clang++"
TOL = 1e-2
CE_TOL = 1e-4


def build(d, sanitize=None):
    sys.path.insert(0, EMU)
    try:
        import prep
    finally:
        sys.path.remove(EMU)
    prep.prepare(CSRC, EMU, d)
    srcs = ["kernels.hip", "attention.hip", "fingerprint.hip", "lib_driver.cpp"]
    flags = ["-g", f"-fsanitize={sanitize}", "-fno-omit-frame-pointer"] if sanitize else []

    def compile_one(src):
        obj = os.path.join(d, src.split(".")[0] + ".o")
        subprocess.run([CLANG, "-std=c++20", "-O1", "-fno-pic", "-w", *flags, "-x", "c++", f"-I{d}", "-c",
                        os.path.join(d, src), "-o", obj], check=True, capture_output=True)
        return obj

    with ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(d, "lib_driver")
    # -no-pie: the static LDS arrays sit below 4 GiB, where the kernels' 32-bit LDS addresses reach them
    subprocess.run([CLANG, "-no-pie", *flags[1:2], *objs, "-o", exe, "-lpthread"], check=True, capture_output=True)
    return exe


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("clang++ not found")
    d = str(tmp_path_factory.mktemp("libemu"))
    return build(d), d


def run(exe, case, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=23",
               TSAN_OPTIONS="halt_on_error=1:exitcode=23")
    subprocess.run([exe, *[str(a) for a in args], case], check=True, timeout=900, env=env)


def f64(u):
    return inputs.bf16_bits_to_f32(u).astype(np.float64)


def put(case, **arrays):
    os.makedirs(case, exist_ok=True)
    for k, a in arrays.items():
        np.ascontiguousarray(a).tofile(os.path.join(case, k + ".bin"))


def get(case, name, dtype, shape):
    a = np.fromfile(os.path.join(case, name + ".bin"), dtype=dtype).reshape(shape)
    return f64(a) if dtype == np.uint16 else a.astype(np.float64)


def plan(exe, d, *shape):
    out = subprocess.run([exe, "plan", *[str(a) for a in shape], d], check=True, capture_output=True,
                         text=True).stdout
    return {line.split()[0]: dict(kv.split("=") for kv in line.split()[1:]) for line in out.splitlines()}


# T, h, f, gelu (0 erf, 1 tanh), bias: ragged tokens and FFN columns, a K tail of 8
# (h = 200), and a token count whose weight gradients are split over K
@pytest.mark.parametrize("T,h,f,gelu,bias", [(300, 128, 264, 0, 1), (600, 200, 264, 1, 0), (1100, 256, 256, 0, 1)])
def test_mlp_shard_emulated(lib, T, h, f, gelu, bias):
    mlp_case(*lib, T, h, f, gelu, bias)


@pytest.mark.parametrize("gelu", [0, 1])
def test_mlp_forward_tail_split_emulated(lib, gelu):
    """The forward plan that splits the last tile columns over K: 257 column tiles
    (one more than the CUs), the last one ragged (136 columns), with a bias; H, Y
    and Z against the oracle, and the split columns on their own."""
    mlp_tail_case(*lib, gelu)


@pytest.mark.parametrize("gelu", [0])
def test_mlp_forward_z_tail_split_emulated(lib, gelu):
    """The forward plan that splits the last tile columns of Z = Y B_i over K:
    257 column tiles of Z (one more than the CUs), the last one ragged (136
    columns); H, Y and Z against the oracle, and Z's split columns on their own."""
    mlp_z_tail_case(*lib, gelu)


def mlp_z_tail_case(exe, d, gelu):
    T, h, f = 200, 256 * 256 + 136, 512
    p = plan(exe, d, T, h, f, 64, 1, 64, 1, 64)["mlp"]
    tn = int(p["z_tail_n"])
    assert tn > 0 and tn % 256 == 136 and int(p["z_tail_splits"]) > 1, p  # the ragged tile is in the tail
    assert p["fwd_tail_n"] == "0", p  # X A_i (two tiles) stays one plain launch
    x = inputs.make_inputs(T, h, f, 64, bias=True)
    case = os.path.join(d, f"mlp_ztail_{gelu}")
    put(case, X=x["X"], A=x["A"], B=x["B"], b1=x["b1"])
    run(exe, case, "mlp_fwd", T, h, f, gelu, 1)
    of = oracle.mlp_shard_fwd(x["X"], x["A"], x["B"], x["b1"], "tanh" if gelu else "erf")
    got = {"H": get(case, "H", np.uint16, (T, f)), "Y": get(case, "Y", np.uint16, (T, f)),
           "Z": get(case, "Z", np.float32, (T, h))}
    errs = {k: rel_fro(v, of[k]) for k, v in got.items()}
    tail = rel_fro(got["Z"][:, -tn:], of["Z"][:, -tn:])
    print(case, errs, tail)
    assert all(e <= TOL for e in list(errs.values()) + [tail]), (errs, tail)


def mlp_tail_case(exe, d, gelu):
    T, h, f = 200, 256, 256 * 256 + 136
    p = plan(exe, d, T, h, f, 64, 1, 64, 1, 64)["mlp"]
    tn = int(p["fwd_tail_n"])
    assert tn > 0 and tn % 256 == 136 and int(p["fwd_tail_splits"]) > 1, p  # the ragged tile is in the tail
    x = inputs.make_inputs(T, h, f, 64, bias=True)
    case = os.path.join(d, f"mlp_tail_{gelu}")
    put(case, X=x["X"], A=x["A"], B=x["B"], b1=x["b1"])
    run(exe, case, "mlp_fwd", T, h, f, gelu, 1)
    of = oracle.mlp_shard_fwd(x["X"], x["A"], x["B"], x["b1"], "tanh" if gelu else "erf")
    got = {"H": get(case, "H", np.uint16, (T, f)), "Y": get(case, "Y", np.uint16, (T, f)),
           "Z": get(case, "Z", np.float32, (T, h))}
    errs = {k: rel_fro(v, of[k]) for k, v in got.items()}
    tail = {k: rel_fro(got[k][:, -tn:], of[k][:, -tn:]) for k in ("H", "Y")}
    print(case, errs, tail)
    assert all(e <= TOL for e in list(errs.values()) + list(tail.values())), (errs, tail)


def mlp_case(exe, d, T, h, f, gelu, bias):
    x = inputs.make_inputs(T, h, f, 64, bias=True)
    case = os.path.join(d, f"mlp_{T}_{h}_{f}_{gelu}_{bias}")
    put(case, X=x["X"], A=x["A"], B=x["B"], dZ=x["dZ"], b1=x["b1"])
    run(exe, case, "mlp_fwd", T, h, f, gelu, bias)
    run(exe, case, "mlp_bwd", T, h, f, gelu, bias)
    form, b1 = ("tanh" if gelu else "erf"), (x["b1"] if bias else None)
    of = oracle.mlp_shard_fwd(x["X"], x["A"], x["B"], b1, form)
    ob = oracle.mlp_shard_bwd(x["X"], x["A"], x["B"], x["dZ"], b1, form)
    got = {"H": get(case, "H", np.uint16, (T, f)), "Y": get(case, "Y", np.uint16, (T, f)),
           "Z": get(case, "Z", np.float32, (T, h)), "dX": get(case, "dX", np.float32, (T, h)),
           "dA": get(case, "dA", np.uint16, (h, f)), "dB": get(case, "dB", np.uint16, (f, h))}
    if bias:
        got["db1"] = get(case, "db1", np.uint16, (f,))
    want = {**of, **ob}
    errs = {k: rel_fro(v, want[k]) for k, v in got.items()}
    print(case, {k: f"{e:.1e}" for k, e in errs.items()})
    assert all(e <= TOL for e in errs.values()), errs


def combine_partials(rng, t, T):
    """Shard partials shaped like real ones: each token's target logit sits in one
    rank's shard and is at most that shard's maximum, and every shard's sum of
    exponentials is at least 2, so each loss is at least ln 2."""
    M = rng.normal(0, 3, (t, T)).astype(np.float32)
    S = rng.uniform(2, 500, (t, T)).astype(np.float32)
    owner = rng.integers(0, t, T)
    Z = np.zeros((t, T), np.float32)
    Z[owner, np.arange(T)] = M[owner, np.arange(T)] - np.abs(rng.normal(0, 3, T)).astype(np.float32)
    return M, S, Z


def fixed_order_mean(loss):
    """The combine's mean in float32: per-thread sums over tokens j, j+1024, ... in
    ascending order, then a binary tree over the 1024 sums, divided by T."""
    T = loss.shape[0]
    acc = np.zeros(1024, np.float32)
    for k in range(0, T, 1024):
        c = loss[k:k + 1024]
        acc[:c.shape[0]] += c
    w = 512
    while w > 0:
        acc[:w] += acc[w:2 * w]
        w //= 2
    return np.float32(acc[0] / np.float32(T))


@pytest.mark.parametrize("T", [3000, 33000])
def test_combine_paths_emulated(lib, T):
    """ce_combine below and above the one-workgroup limit (t*T <= 65536): the loss has
    the same bits whether or not the mean is asked for, and the mean is the fixed-order
    float32 sum of those losses."""
    exe, d = lib
    t = 2
    M, S, Z = combine_partials(np.random.default_rng(11), t, T)
    case = os.path.join(d, f"comb{T}")
    put(case, m=M, s=S, z=Z)
    run(exe, case, "combine", t, T)
    run(exe, case, "combine_nomean", t, T)
    loss = np.fromfile(os.path.join(case, "loss.bin"), np.float32)
    assert np.array_equal(loss.view(np.uint32), np.fromfile(os.path.join(case, "loss_only.bin"), np.uint32))
    oc = oracle.ce_combine(M, S, Z)
    assert np.abs(loss / oc["loss"] - 1).max() <= CE_TOL
    mean = np.fromfile(os.path.join(case, "mean.bin"), np.float32)[0]
    assert mean.view(np.uint32) == fixed_order_mean(loss).view(np.uint32)


def test_vocab_ce_two_shards_emulated(lib):
    """Both ranks' forward partials, the fixed-order combine, and rank 0's backward
    with a per-token upstream gradient (every seventh token weighted 0)."""
    ce_two_shards(*lib)


def ce_two_shards(exe, d):
    T, h, v, t = 300, 128, 520, 2
    case = os.path.join(d, "ce2")
    ms_, ss_, zs_ = [], [], []
    for r in range(t):
        x = inputs.make_inputs(T, h, 64, v, t=t, rank=r)
        put(case, X=x["X"], E=x["E"], target=x["targets"])
        run(exe, case, "ce_fwd", T, h, v, int(x["vocab_start"]))
        o = oracle.vocab_ce_shard(x["X"], x["E"], x["targets"], int(x["vocab_start"]))
        m, s, z = (get(case, k, np.float32, (T,)) for k in ("m", "s", "z"))
        assert np.abs(m - o["m"]).max() <= CE_TOL * np.abs(o["m"]).max()
        assert np.abs(s / o["s"] - 1).max() <= CE_TOL
        assert np.abs(z - o["z"]).max() <= CE_TOL * np.abs(o["z"]).max()
        assert (z[(x["targets"] < r * v) | (x["targets"] >= (r + 1) * v)] == 0).all()
        ms_.append(m), ss_.append(s), zs_.append(z)
    M, S, Zp = (np.stack(a).astype(np.float32) for a in (ms_, ss_, zs_))
    put(case, m=M, s=S, z=Zp)
    run(exe, case, "combine", t, T)
    oc = oracle.ce_combine(M, S, Zp)
    assert np.abs(get(case, "loss", np.float32, (T,)) / oc["loss"] - 1).max() <= CE_TOL
    assert abs(get(case, "mean", np.float32, (1,))[0] / oc["mean"] - 1) <= CE_TOL
    x = inputs.make_inputs(T, h, 64, v, t=t, rank=0)
    dl = np.random.default_rng(5).uniform(0.5, 1.5, T).astype(np.float32)
    dl[::7] = 0
    put(case, X=x["X"], E=x["E"], target=x["targets"], dloss=dl)
    scale = np.float32(1.0 / T)
    run(exe, case, "ce_bwd", T, h, v, 0, t, repr(float(scale)), 1)
    ob = oracle.vocab_ce_shard_bwd(x["X"], x["E"], x["targets"], 0, M, S, float(scale) * dl.astype(np.float64))
    assert rel_fro(get(case, "dX", np.float32, (T, h)), ob["dX"]) <= TOL
    assert rel_fro(get(case, "dE", np.uint16, (h, v)), ob["dE"]) <= TOL


def test_vocab_ce_bwd_split_k_emulated(lib):
    """One shard owning the whole vocabulary, the mean-loss gradient (no dloss), at a
    token count whose dE GEMM is split over K."""
    exe, d = lib
    T, h, v = 1100, 256, 256
    assert int(plan(exe, d, T, h, 256, v, 1, 64, 1, 64)["ce_bwd"]["splits_dE"]) > 1
    x = inputs.make_inputs(T, h, 64, v)
    case = os.path.join(d, "ce1")
    put(case, X=x["X"], E=x["E"], target=x["targets"])
    run(exe, case, "ce_fwd", T, h, v, 0)
    M, S = (get(case, k, np.float32, (T,)).astype(np.float32)[None] for k in ("m", "s"))
    put(case, m=M, s=S)
    scale = np.float32(1.0 / T)
    run(exe, case, "ce_bwd", T, h, v, 0, 1, repr(float(scale)), 0)
    ob = oracle.vocab_ce_shard_bwd(x["X"], x["E"], x["targets"], 0, M, S, float(scale))
    assert rel_fro(get(case, "dX", np.float32, (T, h)), ob["dX"]) <= TOL
    assert rel_fro(get(case, "dE", np.uint16, (h, v)), ob["dE"]) <= TOL


# b, s, h, n, d, causal: the tiny layer, ragged sequences, every head size the
# kernels are built for (32, 64, 96, 128) and the ones padded up to them (16, 48,
# 80, 112), and a token count whose weight gradients are split over K
@pytest.mark.parametrize("b,s,h,n,hd,causal", [
    (2, 32, 64, 4, 16, True), (2, 70, 96, 3, 32, True), (1, 130, 128, 2, 64, False), (1, 96, 192, 2, 96, True),
    (1, 64, 256, 2, 128, False), (3, 1, 64, 2, 32, True), (2, 550, 128, 1, 64, True),
    (1, 150, 96, 2, 48, True), (2, 70, 160, 2, 80, False), (1, 140, 224, 2, 112, True)])
def test_attn_shard_emulated(lib, b, s, h, n, hd, causal):
    attn_case(*lib, b, s, h, n, hd, causal)


@pytest.mark.parametrize("causal", [True, False])
def test_attn_growing_scores_emulated(lib, causal):
    """X row t scaled by 1 + t/32 (as in the GPU test): later key steps raise the forward's running max."""
    attn_case(*lib, 2, 300, 128, 2, 64, causal, grow=1 / 32)


def attn_case(exe, d, b, s, h, n, hd, causal, grow=0.0):
    a = inputs.make_attn_inputs(b, s, h, n, hd)
    if grow:
        f = np.tile(1.0 + grow * np.arange(s), b)[:, None].astype(np.float32)
        a = dict(a, X=inputs.round_to_bf16_bits(inputs.bf16_bits_to_f32(a["X"]) * f))
    case = os.path.join(d, f"attn_{b}_{s}_{h}_{n}_{hd}_{int(causal)}_{grow}")
    put(case, X=a["X"], Wqkv=a["Wqkv"], Wo=a["Wo"], dZ=a["dZ"])
    run(exe, case, "attn_fwd", b, s, h, n, hd, int(causal))
    run(exe, case, "attn_bwd", b, s, h, n, hd, int(causal))
    T, nd = b * s, n * hd
    got = {"QKV": get(case, "QKV", np.uint16, (T, 3 * nd)), "O": get(case, "O", np.uint16, (T, nd)),
           "lse": get(case, "lse", np.float32, (n, T)), "Z": get(case, "Z", np.float32, (T, h)),
           "dX": get(case, "dX", np.float32, (T, h)), "dWqkv": get(case, "dWqkv", np.uint16, (h, 3 * nd)),
           "dWo": get(case, "dWo", np.uint16, (nd, h))}
    want = {**attn.attn_shard_fwd(a["X"], a["Wqkv"], a["Wo"], n, hd, b, s, causal),
            **attn.attn_shard_bwd(a["X"], a["Wqkv"], a["Wo"], a["dZ"], n, hd, b, s, causal)}
    errs = {k: rel_fro(v, want[k]) for k, v in got.items()}
    print(case, {k: f"{e:.1e}" for k, e in errs.items()})
    assert all(e <= TOL for e in errs.values()), errs


def test_emulated_cases_cover_the_plans(lib):
    """The shapes above run both unsplit and split-K weight gradients in every
    backward, and paired launches with either GEMM leading."""
    exe, d = lib
    p_small = plan(exe, d, 300, 128, 264, 520, 2, 70, 3, 32)
    p_split = plan(exe, d, 1100, 256, 256, 256, 2, 550, 1, 64)
    assert p_small["mlp"]["splits_dA"] == "1" and int(p_split["mlp"]["splits_dA"]) > 1
    assert int(p_split["mlp"]["splits_dB"]) > 1
    assert p_small["ce_bwd"]["splits_dE"] == "1"
    assert p_split["attn"]["splits_wqkv"] != "1" or p_split["attn"]["splits_wo"] != "1"
    assert {p_small["mlp"]["dx_first"], p_split["mlp"]["dx_first"]} == {"0", "1"}
    assert p_small["mlp"]["pair_ax"] == "1" and p_small["ce_bwd"]["paired"] == "1"


def _random_case(seed):
    """A seeded random shape for one of the three sequences: any multiple of 8 for
    h, f_i and v_i, any token count, any head size the binding accepts."""
    g = np.random.default_rng(seed)
    kind = ["mlp", "ce", "attn"][seed % 3]
    if kind == "mlp":
        return kind, dict(T=int(g.integers(1, 700)), h=8 * int(g.integers(1, 60)), f=8 * int(g.integers(1, 60)),
                          gelu=int(g.integers(0, 2)), bias=int(g.integers(0, 2)))
    if kind == "ce":
        t = int(g.integers(1, 4))
        return kind, dict(T=int(g.integers(1, 700)), h=8 * int(g.integers(1, 60)), v=8 * int(g.integers(1, 120)),
                          t=t, rank=int(g.integers(0, t)))
    return kind, dict(b=int(g.integers(1, 4)), s=int(g.integers(1, 300)), h=8 * int(g.integers(1, 40)),
                      n=int(g.integers(1, 4)), hd=int(g.choice([16, 32, 48, 64, 80, 96, 112, 128])),
                      causal=bool(g.integers(0, 2)))


@pytest.mark.parametrize("seed", range(100, 112))
def test_random_shapes_emulated(lib, seed):
    """Seeded random shapes through each sequence (the same checks as above): the
    ragged edges, K tails, splits and pairings they happen to hit."""
    exe, d = lib
    kind, p = _random_case(seed)
    print(kind, p)
    if kind == "mlp":
        mlp_case(exe, d, p["T"], p["h"], p["f"], p["gelu"], p["bias"])
    elif kind == "attn":
        attn_case(exe, d, p["b"], p["s"], p["h"], p["n"], p["hd"], p["causal"])
    else:
        T, h, v, t, r = p["T"], p["h"], p["v"], p["t"], p["rank"]
        x = inputs.make_inputs(T, h, 8, v, t=t, rank=r, seed=seed)
        vs = int(x["vocab_start"])
        case = os.path.join(d, f"rand_ce_{seed}")
        put(case, X=x["X"], E=x["E"], target=x["targets"])
        run(exe, case, "ce_fwd", T, h, v, vs)
        o = oracle.vocab_ce_shard(x["X"], x["E"], x["targets"], vs)
        m, s, z = (get(case, k, np.float32, (T,)) for k in ("m", "s", "z"))
        assert np.abs(m - o["m"]).max() <= CE_TOL * np.abs(o["m"]).max()
        assert np.abs(s / o["s"] - 1).max() <= CE_TOL
        assert np.abs(z - o["z"]).max() <= CE_TOL * max(np.abs(o["z"]).max(), 1e-30)
        # the other ranks' partials: this rank's shifted, so the combined statistics differ from the shard's own
        M = np.stack([m + 0.3 * k for k in range(t)]).astype(np.float32)
        S = np.stack([s * (1 + k) for k in range(t)]).astype(np.float32)
        dl = np.random.default_rng(seed).uniform(0, 2, T).astype(np.float32)
        put(case, m=M, s=S, dloss=dl)
        scale = float(np.float32(1.0 / T))
        run(exe, case, "ce_bwd", T, h, v, vs, t, repr(scale), 1)
        ob = oracle.vocab_ce_shard_bwd(x["X"], x["E"], x["targets"], vs, M, S, scale * dl.astype(np.float64))
        assert rel_fro(get(case, "dX", np.float32, (T, h)), ob["dX"]) <= TOL
        assert rel_fro(get(case, "dE", np.uint16, (h, v)), ob["dE"]) <= TOL


@pytest.mark.parametrize("nbytes,chunk", [(0, 64), (100, 32), (70000, 4096), (3 * 65536 + 5, 65536)])
def test_fingerprint_emulated(lib, nbytes, chunk):
    fingerprint_case(*lib, nbytes, chunk)


def fingerprint_case(exe, d, nbytes, chunk):
    from oracle import fingerprint as ofp
    data = np.random.default_rng(nbytes).integers(0, 256, nbytes, dtype=np.uint8)
    case = os.path.join(d, f"fp_{nbytes}_{chunk}")
    put(case, buf=data)
    run(exe, case, "fingerprint", nbytes, chunk)
    got = np.fromfile(os.path.join(case, "fp.bin"), dtype=np.uint64)
    want = ofp.fingerprint(data.tobytes(), chunk)
    assert [int(w) for w in got] == [want["hash"], *want["chunks"]]


@pytest.mark.parametrize("sanitizer", ["address", "thread"])
def test_library_emulated_under_sanitizer(tmp_path, sanitizer):
    """The same launch sequences under a sanitizer; any report stops the run.

    address: every global and LDS access of every kernel stays inside its
    allocation (inputs, outputs and workspaces are allocated at their exact
    sizes, so a read or write past an end is caught; buffer-resource accesses
    are checked against the resource's extent, which must lie inside the
    allocation too).
    thread: every exchange between waves through LDS or memory is ordered by a
    workgroup barrier (each lane is a fiber that the sanitizer tracks like a
    thread, and a wave's lanes meet at each emulated wave-wide operation), and the main loop's vector-memory waits
    land each direct-to-LDS load before its readers' barrier: a wave's loads
    are held back until its own wait requires them, so a missing barrier or a
    too-loose wait shows up as a race on LDS."""
    if not os.path.exists(CLANG):
        pytest.skip("clang++ not found")
    d = str(tmp_path)
    exe = build(d, sanitize=sanitizer)
    mlp_case(exe, d, 600, 200, 264, 1, 0)
    ce_two_shards(exe, d)
    attn_case(exe, d, 2, 70, 96, 3, 32, True)
    if sanitizer == "address":
        attn_case(exe, d, 3, 1, 64, 2, 32, True)
        fingerprint_case(exe, d, 100, 32)
        fingerprint_case(exe, d, 0, 64)
    else:
        attn_case(exe, d, 1, 130, 128, 2, 64, False)
        fingerprint_case(exe, d, 70000, 4096)


FULL = os.environ.get("MSHARD_FULL_SIZE_EMULATION") == "1"


@pytest.mark.skipif(not FULL, reason="about a minute; set MSHARD_FULL_SIZE_EMULATION=1")
def test_mlp_forward_tail_split_under_address_sanitizer(lib_asan):
    """The forward's split tails (GEMM slices and their GeLU and fp32 reductions)
    with every access checked against its allocation."""
    mlp_tail_case(*lib_asan, 0)
    mlp_z_tail_case(*lib_asan, 0)


@pytest.fixture(scope="module")
def lib_asan(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("clang++ not found")
    d = str(tmp_path_factory.mktemp("libemu_asan"))
    return build(d, sanitize="address"), d


def sampled_rel_fro(got, want_fn):
    """Relative Frobenius error over the entries the sampled workgroups wrote
    (the others stay NaN); want_fn(rows, cols) gives the oracle on that grid."""
    ok = ~np.isnan(got)
    rows, cols = np.nonzero(ok.any(axis=1))[0], np.nonzero(ok.any(axis=0))[0]
    assert len(rows) and len(cols)
    want = want_fn(rows, cols)
    sub, msk = got[np.ix_(rows, cols)], ok[np.ix_(rows, cols)]
    return np.linalg.norm((sub - want)[msk]) / np.linalg.norm(want[msk]), want, sub, msk


@pytest.mark.skipif(not FULL, reason="minutes of CPU and up to 8 GB of memory: set MSHARD_FULL_SIZE_EMULATION=1")
@pytest.mark.parametrize("name", ["gpt2_1p5b", "gpt_8p3b_t8", "bert_3p9b_t4", "bloom_176b_t4"])
def test_full_size_sampled_under_address_sanitizer(lib_asan, name):
    """The CE backward and the attention shard at each workload's real shard shape,
    under AddressSanitizer, with every GEMM and attention-core launch cut down to
    six of its workgroups (two at each end of its workgroup order, two between;
    the small per-token kernels run in full).  Every launch of both sequences
    runs with the real grids, strides and workspace layout, and no access leaves
    its allocation.  The values of the first stage of each sequence are checked
    where the sampled workgroups wrote them: the logit gradient dL (with given
    row statistics, so that its softmax term is not negligible), the QKV
    projection, and the attention core's output on random full-size QKV."""
    exe, d = lib_asan
    env = dict(os.environ, EMU_SAMPLE="2", EMU_WRITE_DL="1")

    def go(case, *args):
        subprocess.run([exe, *[str(a) for a in args], case], check=True, timeout=3000,
                       env=dict(env, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=23"))

    # vocab-parallel CE backward of rank 0
    c = inputs.CONFIGS[name]
    x = inputs.make_config_inputs(c, want=("X", "E", "targets"))
    T, h, v, t = c.T, c.h, c.v_i, c.t
    g = np.random.default_rng(7)
    m = (0.1 * g.standard_normal((t, T))).astype(np.float32)
    s = (20 * (1 + 0.1 * g.random((t, T)))).astype(np.float32)
    case = os.path.join(d, f"full_ce_{name}")
    put(case, X=x["X"], E=x["E"], target=x["targets"], m=m, s=s)
    scale = float(np.float32(1.0 / T))
    go(case, "ce_bwd", T, h, v, 0, t, repr(scale), 0)
    st = oracle.ce_row_stats(m, s)
    err, want, sub, msk = sampled_rel_fro(
        get(case, "dL", np.uint16, (T, v)),
        lambda r, cl: oracle.ref._ce_grad_block(f64(x["X"][r]) @ f64(x["E"][:, cl]), st["M"][r], st["S"][r],
                                                np.full(len(r), scale), x["targets"][r], 0, cl))
    soft = msk & (want > 0)
    assert err <= TOL
    assert np.linalg.norm((sub - want)[soft]) / np.linalg.norm(want[soft]) <= TOL
    del x
    subprocess.run(["rm", "-rf", case], check=True)

    # attention shard, and its core alone on random full-size QKV
    a_cfg = inputs.ATTN_CONFIGS[name]
    b, sq, hh, n, hd, causal = a_cfg.b, a_cfg.s, a_cfg.h, a_cfg.n, a_cfg.d, a_cfg.causal
    a = inputs.make_attn_config_inputs(a_cfg)
    case = os.path.join(d, f"full_attn_{name}")
    put(case, X=a["X"], Wqkv=a["Wqkv"], Wo=a["Wo"], dZ=a["dZ"])
    go(case, "attn_fwd", b, sq, hh, n, hd, int(causal))
    go(case, "attn_bwd", b, sq, hh, n, hd, int(causal))
    T, nd = b * sq, n * hd
    err = sampled_rel_fro(get(case, "QKV", np.uint16, (T, 3 * nd)),
                          lambda r, cl: f64(a["X"][r]) @ f64(a["Wqkv"][:, cl]))[0]
    assert err <= TOL
    subprocess.run(["rm", "-rf", case], check=True)
    g = np.random.default_rng(3)
    q = inputs.round_to_bf16_bits(g.standard_normal((T, 3 * nd)).astype(np.float32))
    do = inputs.round_to_bf16_bits(g.standard_normal((T, nd)).astype(np.float32))
    case = os.path.join(d, f"full_core_{name}")
    put(case, qkv=q, dout=do)
    go(case, "attn_core", b, sq, n, hd, int(causal))
    O = get(case, "o", np.uint16, (T, nd))
    Q, K, V = f64(q[:, :nd]), f64(q[:, nd:2 * nd]), f64(q[:, 2 * nd:])
    pairs = 0
    for bi in range(b):
        for j in range(n):
            rs, cs = slice(bi * sq, (bi + 1) * sq), slice(j * hd, (j + 1) * hd)
            okr = ~np.isnan(O[rs, cs]).any(axis=1)
            if okr.any():
                w = attn.attention_core(Q[rs, cs], K[rs, cs], V[rs, cs], 1, hd, 1, sq, causal)["O"]
                assert rel_fro(O[rs, cs][okr], w[okr]) <= TOL
                pairs += 1
    assert pairs > 0
    subprocess.run(["rm", "-rf", case], check=True)


def _scaled_bf16(u, k):
    """bf16 bit patterns times 2**k (exact: only the exponent moves)."""
    return inputs.round_to_bf16_bits(inputs.bf16_bits_to_f32(u) * np.float32(2.0 ** k))


def test_vocab_ce_degenerate_and_extreme_logits(lib):
    """E = 0: every logit is 0, so m = 0, s = v_i and z = 0 exactly, and the
    gradient is coef (1/v - one-hot) with dE = X^T dL.  Logits 64 times larger
    than the workloads' (std about 50): the shard max is subtracted before every
    exponential, so nothing overflows and the partials keep their relative
    accuracy."""
    exe, d = lib
    T, h, v = 300, 128, 520
    x = inputs.make_inputs(T, h, 8, v)
    case = os.path.join(d, "ce_zero")
    put(case, X=x["X"], E=np.zeros_like(x["E"]), target=x["targets"])
    run(exe, case, "ce_fwd", T, h, v, 0)
    m, s, z = (get(case, k, np.float32, (T,)) for k in ("m", "s", "z"))
    assert (m == 0).all() and (s == v).all() and (z == 0).all()
    put(case, m=m.astype(np.float32)[None], s=s.astype(np.float32)[None])
    run(exe, case, "ce_bwd", T, h, v, 0, 1, repr(float(np.float32(1.0 / T))), 0)
    ob = oracle.vocab_ce_shard_bwd(x["X"], np.zeros_like(x["E"]), x["targets"], 0, m[None], s[None], 1.0 / T)
    assert rel_fro(get(case, "dE", np.uint16, (h, v)), ob["dE"]) <= TOL
    assert np.abs(get(case, "dX", np.float32, (T, h))).max() == 0

    Xb = _scaled_bf16(x["X"], 6)
    case = os.path.join(d, "ce_big")
    put(case, X=Xb, E=x["E"], target=x["targets"])
    run(exe, case, "ce_fwd", T, h, v, 0)
    o = oracle.vocab_ce_shard(Xb, x["E"], x["targets"], 0)
    m, s, z = (get(case, k, np.float32, (T,)) for k in ("m", "s", "z"))
    # the max logit's own term is exp of the rounding error of m log2(e) (about 1e-5 here), so s may sit just below 1
    assert np.isfinite(m).all() and np.isfinite(s).all() and (s > 0.999).all()
    assert np.abs(m - o["m"]).max() <= CE_TOL * np.abs(o["m"]).max()
    assert np.abs(s / o["s"] - 1).max() <= CE_TOL
    put(case, m=m.astype(np.float32)[None], s=s.astype(np.float32)[None])
    run(exe, case, "ce_bwd", T, h, v, 0, 1, repr(float(np.float32(1.0 / T))), 0)
    ob = oracle.vocab_ce_shard_bwd(Xb, x["E"], x["targets"], 0, m[None], s[None], 1.0 / T)
    assert rel_fro(get(case, "dX", np.float32, (T, h)), ob["dX"]) <= TOL
    assert rel_fro(get(case, "dE", np.uint16, (h, v)), ob["dE"]) <= TOL


@pytest.mark.parametrize("causal", [True, False])
def test_attention_core_uniform_and_peaked(lib, causal):
    """Q = 0: every visible key has the same score, so each query's output is the
    mean of the values it sees and lse = ln(visible keys).  Scores 16 times the
    usual scale (Q times 16): softmax rows close to one-hot, where the running
    max of the online softmax matters most."""
    exe, d = lib
    b, s, n, hd = 2, 150, 2, 64
    T, nd = b * s, n * hd
    g = np.random.default_rng(9)
    qkv = inputs.round_to_bf16_bits(g.standard_normal((T, 3 * nd)).astype(np.float32))
    dout = inputs.round_to_bf16_bits(g.standard_normal((T, nd)).astype(np.float32))
    zero_q = qkv.copy()
    zero_q[:, :nd] = 0
    case = os.path.join(d, f"core_uniform_{int(causal)}")
    put(case, qkv=zero_q, dout=dout)
    run(exe, case, "attn_core", b, s, n, hd, int(causal))
    O = get(case, "o", np.uint16, (T, nd))
    lse = get(case, "lse", np.float32, (n, T))
    V = f64(zero_q[:, 2 * nd:])
    want = np.empty((T, nd))
    vis = np.empty(T)
    for bi in range(b):
        for q in range(s):
            k_end = q + 1 if causal else s
            want[bi * s + q] = V[bi * s:bi * s + k_end].mean(axis=0)
            vis[bi * s + q] = k_end
    assert rel_fro(O, want) <= TOL
    assert np.abs(lse - np.log(vis)[None, :]).max() <= 1e-5

    peaked = qkv.copy()
    peaked[:, :nd] = _scaled_bf16(qkv[:, :nd], 4)
    case = os.path.join(d, f"core_peaked_{int(causal)}")
    put(case, qkv=peaked, dout=dout)
    run(exe, case, "attn_core", b, s, n, hd, int(causal))
    Q, K, V = f64(peaked[:, :nd]), f64(peaked[:, nd:2 * nd]), f64(peaked[:, 2 * nd:])
    want = attn.attention_core(Q, K, V, n, hd, b, s, causal)
    assert rel_fro(get(case, "o", np.uint16, (T, nd)), want["O"]) <= TOL
    assert rel_fro(get(case, "lse", np.float32, (n, T)), want["lse"]) <= 1e-5
    qt, kt, vt = (torch.tensor(x.reshape(b, s, n, hd).transpose(0, 2, 1, 3).copy(), requires_grad=True)
                  for x in (Q, K, V))
    ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    (ot * torch.tensor(f64(dout).reshape(b, s, n, hd).transpose(0, 2, 1, 3).copy())).sum().backward()
    dq = get(case, "dqkv", np.uint16, (T, 3 * nd))
    for j, t in enumerate((qt, kt, vt)):
        assert rel_fro(dq[:, j * nd:(j + 1) * nd], t.grad.numpy().transpose(0, 2, 1, 3).reshape(T, nd)) <= TOL


@pytest.mark.parametrize("gelu", [0, 1])
def test_mlp_degenerate_and_extreme_inputs(lib, gelu):
    """A = 0 with a bias: every H row equals b1, so Y rows are GeLU(b1) and
    dX = dH A^T is exactly 0.  X 1024 times the workloads' scale (|H| in the
    hundreds): the exponential in GeLU and GeLU' underflows to 0, leaving
    max(x, 0) and the step function, with no NaN from the products."""
    exe, d = lib
    T, h, f = 300, 136, 264
    x = inputs.make_inputs(T, h, f, 8, bias=True)
    form = "tanh" if gelu else "erf"
    for label, X, A in (("zeroA", x["X"], np.zeros_like(x["A"])), ("bigX", _scaled_bf16(x["X"], 10), x["A"])):
        case = os.path.join(d, f"mlp_{label}_{gelu}")
        put(case, X=X, A=A, B=x["B"], dZ=x["dZ"], b1=x["b1"])
        run(exe, case, "mlp_fwd", T, h, f, gelu, 1)
        run(exe, case, "mlp_bwd", T, h, f, gelu, 1)
        of = oracle.mlp_shard_fwd(X, A, x["B"], x["b1"], form)
        ob = oracle.mlp_shard_bwd(X, A, x["B"], x["dZ"], x["b1"], form)
        got = {"H": get(case, "H", np.uint16, (T, f)), "Y": get(case, "Y", np.uint16, (T, f)),
               "Z": get(case, "Z", np.float32, (T, h)), "dA": get(case, "dA", np.uint16, (h, f)),
               "dB": get(case, "dB", np.uint16, (f, h)), "db1": get(case, "db1", np.uint16, (f,))}
        dX = get(case, "dX", np.float32, (T, h))
        for k, v in got.items():
            assert np.isfinite(v).all() and rel_fro(v, {**of, **ob}[k]) <= TOL, (label, k)
        if label == "zeroA":
            assert (got["H"] == got["H"][0][None, :]).all()
            assert np.abs(dX).max() == 0
        else:
            assert np.isfinite(dX).all() and rel_fro(dX, ob["dX"]) <= TOL
