"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances: relative Frobenius error <= 1e-2 for every bf16-input GEMM output
and gradient (H_i, Y_i, Z_i, dX_i, dA_i, dB_i, db1_i); <= 1e-4 relative for the
CE partials (m, s, z), the per-token loss (max relative) and the mean loss.

Sizes: full comparisons at sizes the oracle finishes in seconds (a tiny layer,
and ragged shapes spanning several 256-wide tiles, a K tail and split-K weight
gradients); at the four large workloads' full sizes, sampled token rows and
FFN columns that the oracle evaluates one by one (tile-edge indices always
included) for the MLP, and every token for the vocab-parallel CE.  Bitwise
determinism at the benchmark's shape, with a concurrent stream.
"""
import hashlib

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_mlp_amd import inputs
from tests.conftest import rel_fro

pytestmark = pytest.mark.gpu

MLP_TOL = 1e-2
CE_TOL = 1e-4


@pytest.fixture(scope="module")
def ms():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from megatron_tensor_transformer_mlp_amd import mshard
    return mshard


def dev(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return inputs.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.double().cpu().numpy()


def digest(*ts) -> str:
    h = hashlib.sha256()
    for t in ts:
        h.update(t.contiguous().view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


def run_mlp(ms, d, gelu="erf", bias=False):
    X, A, B, dZ = dev(d["X"]), dev(d["A"]), dev(d["B"]), dev(d["dZ"])
    b1 = dev(d["b1"]) if bias else None
    H, Y, Z = ms.mlp_shard_fwd(X, A, B, b1, gelu=gelu)
    dX, dA, dB, db1 = ms.mlp_shard_bwd(X, A, B, H, Y, dZ, gelu=gelu, want_db1=bias)
    torch.cuda.synchronize()
    return dict(H=H, Y=Y, Z=Z, dX=dX, dA=dA, dB=dB, db1=db1)


def check_mlp_full(g, d, gelu, bias):
    b1 = d["b1"] if bias else None
    of = oracle.mlp_shard_fwd(d["X"], d["A"], d["B"], b1, gelu)
    ob = oracle.mlp_shard_bwd(d["X"], d["A"], d["B"], d["dZ"], b1, gelu)
    errs = {k: rel_fro(host(g[k]), of[k]) for k in ("H", "Y", "Z")}
    errs.update({k: rel_fro(host(g[k]), ob[k]) for k in ("dX", "dA", "dB")})
    if bias:
        errs["db1"] = rel_fro(host(g["db1"]), ob["db1"])
    print("mlp rel-fro errors:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= MLP_TOL, (k, v)
    return errs


def run_ce(ms, d):
    m, s, z = ms.vocab_ce_shard_fwd(dev(d["X"]), dev(d["E"]), torch.from_numpy(d["targets"]).cuda(),
                                    int(d["vocab_start"]))
    torch.cuda.synchronize()
    return m, s, z


def check_ce_full(ms, d):
    m, s, z = run_ce(ms, d)
    o = oracle.vocab_ce_shard(d["X"], d["E"], d["targets"], int(d["vocab_start"]))
    for name, got in (("m", m), ("s", s), ("z", z)):
        e = rel_fro(host(got), o[name])
        print(f"ce {name} rel-fro {e:.2e}", flush=True)
        assert e <= CE_TOL, (name, e)
    return m, s, z


# ----------------------------------------------------------------------------- full comparisons
@pytest.mark.parametrize("gelu", ["erf", "tanh"])
@pytest.mark.parametrize("bias", [False, True])
def test_tiny_layer_full(ms, gelu, bias):
    """Tiny full layer: T=64, h=64, ffn 256, vocab 512 (t=1)."""
    c = inputs.CONFIGS["tiny"]
    d = inputs.make_inputs(c.T, c.h, c.f_i, c.v_i, bias=bias)
    print(f"case tiny gelu={gelu} bias={bias}", flush=True)
    check_mlp_full(run_mlp(ms, d, gelu, bias), d, gelu, bias)
    m, s, z = check_ce_full(ms, d)
    loss, mean = ms.ce_combine(m[None], s[None], z[None])
    want = oracle.full_vocab_ce(d["X"], d["E"], d["targets"])
    assert np.max(np.abs(host(loss) - want) / np.abs(want)) <= CE_TOL
    assert abs(host(mean)[0] - want.mean()) <= CE_TOL * abs(want.mean())


@pytest.mark.parametrize("T,h,f,v", [(600, 392, 776, 1000), (4100, 392, 776, 1000), (1, 8, 8, 8), (37, 72, 24, 40)])
def test_ragged_full(ms, T, h, f, v):
    """Shapes with ragged M/N tails, a K tail (h % 64 != 0), several tiles, and
    (T=4100) split-K weight gradients; plus single-token and sub-tile shapes."""
    d = inputs.make_inputs(T, h, f, v, t=2, rank=1, v_global=2 * v, bias=True)
    print(f"case ragged T={T} h={h} f={f} v={v}", flush=True)
    check_mlp_full(run_mlp(ms, d, "erf", True), d, "erf", True)
    check_ce_full(ms, d)


# ----------------------------------------------------------------------------- full-size sampled
BIG = ["gpt2_1p5b", "gpt_8p3b_t8", "bert_3p9b_t4", "bloom_176b_t4"]


def _sample(c):
    rows = inputs.sample_indices(c.T, 256, 11, [0, 127, 128, 255, 256, c.T - 1])
    cols = inputs.sample_indices(c.f_i, 256, 12, [0, 63, 64, 127, 128, 255, 256, c.f_i - 1])
    return rows, cols


@pytest.mark.parametrize("name", BIG)
def test_mlp_full_size_sampled(ms, name):
    c = inputs.CONFIGS[name]
    print(f"case mlp {name} T={c.T} h={c.h} f_i={c.f_i}", flush=True)
    d = inputs.make_config_inputs(c, want=("X", "A", "B", "dZ"))
    g = run_mlp(ms, d)
    rows, cols = _sample(c)
    o = oracle.mlp_shard_sampled(d["X"], d["A"], d["B"], d["dZ"], rows, cols)
    R = torch.from_numpy(rows).cuda()
    C = torch.from_numpy(cols).cuda()
    errs = {
        "H": rel_fro(host(g["H"][R]), o["H_rows"]),
        "Y": rel_fro(host(g["Y"][R]), o["Y_rows"]),
        "Z": rel_fro(host(g["Z"][R]), o["Z_rows"]),
        "dX": rel_fro(host(g["dX"][R]), o["dX_rows"]),
        "dA": rel_fro(host(g["dA"][:, C]), o["dA_cols"]),
        "dB": rel_fro(host(g["dB"][C, :]), o["dB_cols"]),
    }
    print(name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= MLP_TOL, (k, v)


@pytest.mark.parametrize("name", BIG)
def test_ce_full_size(ms, name):
    """All t vocab shards on the GPU, combined on the GPU.  The oracle evaluates
    every shard's partials over all T tokens: shard 0's (m, s, z), the per-token
    loss of every token and the mean over all T tokens are compared with it
    (at most 1.5e13 fp64 flops, the 176B-scale layer)."""
    c = inputs.CONFIGS[name]
    print(f"case ce {name} T={c.T} h={c.h} v_i={c.v_i} t={c.t}", flush=True)
    base = inputs.make_config_inputs(c, want=("X", "targets"))
    X = dev(base["X"])
    tg = torch.from_numpy(base["targets"]).cuda()
    ms_, ss_, zs_ = [], [], []
    o_m, o_s, o_z = [], [], []
    for r in range(c.t):
        E = inputs.make_config_inputs(c, rank=r, want=("E",))["E"]
        m, s, z = ms.vocab_ce_shard_fwd(X, dev(E), tg, r * c.v_i)
        ms_.append(m); ss_.append(s); zs_.append(z)
        o = oracle.vocab_ce_shard(base["X"], E, base["targets"], r * c.v_i)
        o_m.append(o["m"]); o_s.append(o["s"]); o_z.append(o["z"])
        if r == 0:
            for k, got in (("m", m), ("s", s), ("z", z)):
                e = rel_fro(host(got), o[k])
                print(f"  shard0 {k} rel-fro {e:.2e}", flush=True)
                assert e <= CE_TOL, (k, e)
        del E
    loss, mean = ms.ce_combine(torch.stack(ms_), torch.stack(ss_), torch.stack(zs_))
    torch.cuda.synchronize()
    want = oracle.ce_combine(o_m, o_s, o_z)
    gl = host(loss)
    err = np.max(np.abs(gl - want["loss"]) / np.abs(want["loss"]))
    gmean = host(mean)[0]
    merr = abs(gmean - want["mean"]) / abs(want["mean"])
    print(f"  loss max-rel {err:.2e} over {c.T} tokens; mean {gmean:.6f} vs oracle {want['mean']:.6f}"
          f" (rel {merr:.2e}; ln v = {np.log(c.v_global):.6f})", flush=True)
    assert err <= CE_TOL
    assert merr <= CE_TOL


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


@pytest.mark.parametrize("gelu", ["erf", "tanh"])
def test_forward_tail_split(ms, gelu):
    """A shape whose forward splits its last tile columns over K (264 tiles on 256
    CUs): H, Y and Z against the oracle, the split columns on their own, the
    backward from those H and Y, and the same bits on a second call."""
    T, h, f = 2048, 512, 8448
    assert ms.mlp_shard_fwd_workspace_bytes(T, h, f) > 0
    print(f"case forward tail split gelu={gelu} T={T} h={h} f={f}", flush=True)
    d = inputs.make_inputs(T, h, f, 8, bias=True)
    X, A, B, dZ, b1 = dev(d["X"]), dev(d["A"]), dev(d["B"]), dev(d["dZ"]), dev(d["b1"])
    H, Y, Z = ms.mlp_shard_fwd(X, A, B, b1, gelu=gelu)
    H2, Y2, Z2 = ms.mlp_shard_fwd(X, A, B, b1, gelu=gelu)
    dX, dA, dB, db1 = ms.mlp_shard_bwd(X, A, B, H, Y, dZ, gelu=gelu, want_db1=True)
    torch.cuda.synchronize()
    assert digest(H, Y, Z) == digest(H2, Y2, Z2)
    want = {**oracle.mlp_shard_fwd(d["X"], d["A"], d["B"], d["b1"], gelu),
            **oracle.mlp_shard_bwd(d["X"], d["A"], d["B"], d["dZ"], d["b1"], gelu)}
    got = {"H": host(H), "Y": host(Y), "Z": host(Z), "dX": host(dX), "dA": host(dA), "dB": host(dB),
           "db1": host(db1)}
    errs = {k: rel_fro(v, want[k]) for k, v in got.items()}
    errs.update({k + "_tail": rel_fro(got[k][:, -256:], want[k][:, -256:]) for k in ("H", "Y")})
    print("  rel-fro", {k: f"{e:.2e}" for k, e in errs.items()}, flush=True)
    assert all(e <= MLP_TOL for e in errs.values()), errs


def test_forward_z_tail_split(ms):
    """A shape whose forward splits the last tile columns of Z = Y B_i over K
    (264 tiles of Z on 256 CUs): H, Y and Z against the oracle, Z's split
    columns on their own, and the same bits on a second call."""
    T, h, f = 2048, 8448, 512
    assert ms.mlp_shard_fwd_workspace_bytes(T, h, f) > 0
    print(f"case forward Z tail split T={T} h={h} f={f}", flush=True)
    d = inputs.make_inputs(T, h, f, 8, bias=True)
    X, A, B, b1 = dev(d["X"]), dev(d["A"]), dev(d["B"]), dev(d["b1"])
    H, Y, Z = ms.mlp_shard_fwd(X, A, B, b1)
    H2, Y2, Z2 = ms.mlp_shard_fwd(X, A, B, b1)
    torch.cuda.synchronize()
    assert digest(H, Y, Z) == digest(H2, Y2, Z2)
    want = oracle.mlp_shard_fwd(d["X"], d["A"], d["B"], d["b1"], "erf")
    got = {"H": host(H), "Y": host(Y), "Z": host(Z)}
    errs = {k: rel_fro(v, want[k]) for k, v in got.items()}
    errs["Z_tail"] = rel_fro(got["Z"][:, -256:], want["Z"][:, -256:])
    print("  rel-fro", {k: f"{e:.2e}" for k, e in errs.items()}, flush=True)
    assert all(e <= MLP_TOL for e in errs.values()), errs


def fixed_order_mean(loss: np.ndarray) -> np.float32:
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


@pytest.mark.parametrize("t,T", [(1, 8192), (8, 8192), (2, 33000), (3, 100000)])
def test_combine_paths(ms, t, T):
    """ce_combine at and above the one-workgroup limit (t*T <= 65536): the loss has the
    same bits with and without the mean, it matches the oracle, and the mean is the
    fixed-order float32 sum of those losses, bit for bit."""
    M, S, Z = combine_partials(np.random.default_rng(17 + t), t, T)
    print(f"  ce_combine t={t} T={T}", flush=True)
    m, s, z = (torch.from_numpy(a).cuda() for a in (M, S, Z))
    loss, mean = ms.ce_combine(m, s, z)
    loss_only, none = ms.ce_combine(m, s, z, want_mean=False)
    torch.cuda.synchronize()
    assert none is None
    gl = loss.cpu().numpy()
    assert torch.equal(loss.view(torch.int32), loss_only.view(torch.int32))
    want = oracle.ce_combine(M, S, Z)
    assert np.max(np.abs(gl / want["loss"] - 1)) <= CE_TOL
    assert mean.cpu().numpy()[0].view(np.uint32) == fixed_order_mean(gl).view(np.uint32)


# ----------------------------------------------------------------------------- determinism
def test_bitwise_determinism(ms):
    """Repeated calls on identical inputs give identical output bytes, also with
    freshly allocated output buffers and a dirty workspace."""
    d = inputs.make_inputs(4100, 392, 776, 1000, bias=True)
    X, A, B, dZ, b1 = dev(d["X"]), dev(d["A"]), dev(d["B"]), dev(d["dZ"]), dev(d["b1"])
    E, tg = dev(d["E"]), torch.from_numpy(d["targets"]).cuda()
    ref = None
    for it in range(10):
        ws = torch.full((ms.mlp_shard_workspace_bytes(4100, 392, 776),), it, dtype=torch.uint8, device="cuda")
        H, Y, Z = ms.mlp_shard_fwd(X, A, B, b1)
        dX, dA, dB, db1 = ms.mlp_shard_bwd(X, A, B, H, Y, dZ, want_db1=True, workspace=ws)
        m, s, z = ms.vocab_ce_shard_fwd(X, E, tg, 0)
        loss, mean = ms.ce_combine(m[None], s[None], z[None])
        h = digest(H, Y, Z, dX, dA, dB, db1, m, s, z, loss, mean)
        ref = ref or h
        assert h == ref, it


def test_bitwise_determinism_bench_shape_concurrent(ms):
    """At the GPT-2 1.5B-like layer, the shape the benchmark times (its backward
    runs (dB, dH) as one paired launch), every entry point of the step gives
    identical bytes over 12 runs: dirty workspaces filled differently each run,
    fresh outputs, and on every other run a stream of unrelated GEMMs running
    at the same time on a second stream, so the library's workgroups share the
    CUs with another kernel in a different order each time."""
    c = inputs.CONFIGS["gpt2_1p5b"]
    d = inputs.make_config_inputs(c)
    X, A, B, dZ, E = dev(d["X"]), dev(d["A"]), dev(d["B"]), dev(d["dZ"]), dev(d["E"])
    tg = torch.from_numpy(d["targets"]).cuda()
    side = torch.cuda.Stream()
    busy_a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    busy_b = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    nbytes = {"mlp": ms.mlp_shard_workspace_bytes(c.T, c.h, c.f_i),
              "ce": ms.vocab_ce_workspace_bytes(c.T, c.h, c.v_i),
              "ce_bwd": ms.vocab_ce_bwd_workspace_bytes(c.T, c.h, c.v_i)}
    ref = None
    for it in range(12):
        ws = {k: torch.full((n,), 17 * it + 3, dtype=torch.uint8, device="cuda") for k, n in nbytes.items()}
        torch.cuda.synchronize()
        if it % 2:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(40):
                    busy_c = busy_a @ busy_b
        H, Y, Z = ms.mlp_shard_fwd(X, A, B)
        dX, dA, dB, _ = ms.mlp_shard_bwd(X, A, B, H, Y, dZ, workspace=ws["mlp"])
        m, s, z = ms.vocab_ce_shard_fwd(X, E, tg, 0, workspace=ws["ce"])
        loss, mean = ms.ce_combine(m[None], s[None], z[None])
        cdX, cdE = ms.vocab_ce_shard_bwd(X, E, tg, m[None], s[None], 0, workspace=ws["ce_bwd"])
        torch.cuda.synchronize()
        outs = dict(H=H, Y=Y, Z=Z, dX=dX, dA=dA, dB=dB, m=m, s=s, z=z, loss=loss, mean=mean, ce_dX=cdX, ce_dE=cdE)
        h = {k: digest(v)[:16] for k, v in outs.items()}
        print(f"  run {it} {'with' if it % 2 else 'without'} a concurrent stream: {h}", flush=True)
        ref = ref or h
        assert h == ref, (it, sorted(k for k in h if h[k] != ref[k]))
    del busy_c


# ----------------------------------------------------------------------------- multi-rank emulation
@pytest.mark.parametrize("t", [2, 4])
def test_tensor_parallel_emulation(ms, t):
    """Run all t rank shards sequentially on one GPU: the sum of the Z_r partials
    (what g would all-reduce) and of the dX_r partials (what f would all-reduce)
    match the unsharded layer, and the combined vocab shards match full-vocab CE."""
    T, h, f, v = 512, 256, 1024, 2048
    d = inputs.make_inputs(T, h, f, v)
    X, dZ = dev(d["X"]), dev(d["dZ"])
    fs, vs = f // t, v // t
    Zs, dXs, mss, sss, zss = 0, 0, [], [], []
    tg = torch.from_numpy(d["targets"]).cuda()
    for r in range(t):
        A_r = dev(np.ascontiguousarray(d["A"][:, r * fs:(r + 1) * fs]))
        B_r = dev(np.ascontiguousarray(d["B"][r * fs:(r + 1) * fs, :]))
        H, Y, Z = ms.mlp_shard_fwd(X, A_r, B_r)
        dX, dA, dB, _ = ms.mlp_shard_bwd(X, A_r, B_r, H, Y, dZ)
        Zs = Zs + host(Z)
        dXs = dXs + host(dX)
        E_r = dev(np.ascontiguousarray(d["E"][:, r * vs:(r + 1) * vs]))
        m, s, z = ms.vocab_ce_shard_fwd(X, E_r, tg, r * vs)
        mss.append(m); sss.append(s); zss.append(z)
    of = oracle.mlp_shard_fwd(d["X"], d["A"], d["B"])
    ob = oracle.mlp_shard_bwd(d["X"], d["A"], d["B"], d["dZ"])
    assert rel_fro(Zs, of["Z"]) <= MLP_TOL
    assert rel_fro(dXs, ob["dX"]) <= MLP_TOL
    loss, mean = ms.ce_combine(torch.stack(mss), torch.stack(sss), torch.stack(zss))
    want = oracle.full_vocab_ce(d["X"], d["E"], d["targets"])
    assert np.max(np.abs(host(loss) - want) / np.abs(want)) <= CE_TOL
    assert abs(host(mean)[0] - want.mean()) <= CE_TOL * abs(want.mean())


def test_ce_target_ownership_edges(ms):
    """Targets exactly at this shard's first/last column, just outside it, and a
    shard that owns none of the targets (z must be exactly 0 there)."""
    T, h, v = 300, 136, 520
    d = inputs.make_inputs(T, h, 8, v, t=3, rank=1, v_global=3 * v)
    start = int(d["vocab_start"])
    tg = d["targets"].copy()
    tg[:6] = [start, start + v - 1, start - 1, start + v, start + 255, start + 256]
    d["targets"] = tg
    m, s, z = check_ce_full(ms, d)
    zh = host(z)
    assert zh[2] == 0.0 and zh[3] == 0.0
    d2 = dict(d)
    d2["targets"] = np.zeros(T, dtype=np.int64)  # all owned by rank 0
    _, _, z2 = run_ce(ms, d2)
    assert not host(z2).any()


# ----------------------------------------------------------------------------- degenerate and extreme inputs
# A = 0 with a bias: every H row equals b1, Y rows are GeLU(b1), dX is exactly 0.
# X 1024 times the workloads' scale: GeLU and GeLU' reduce to max(x, 0) and a
# step, and nothing may turn into NaN.
@pytest.mark.parametrize("gelu", ["erf", "tanh"])
@pytest.mark.parametrize("label", ["zeroA", "bigX"])
def test_mlp_edges(ms, gelu, label):
    T, h, f = 300, 136, 264
    print(f"case mlp edges {label} gelu={gelu} T={T} h={h} f={f}", flush=True)
    x = inputs.make_inputs(T, h, f, 8, bias=True)
    X, A = x["X"], x["A"]
    if label == "zeroA":
        A = np.zeros_like(A)
    else:
        X = inputs.round_to_bf16_bits(inputs.bf16_bits_to_f32(X) * np.float32(1024.0))
    H, Y, Z = ms.mlp_shard_fwd(dev(X), dev(A), dev(x["B"]), dev(x["b1"]), gelu=gelu)
    dX, dA, dB, db1 = ms.mlp_shard_bwd(dev(X), dev(A), dev(x["B"]), H, Y, dev(x["dZ"]), gelu=gelu, want_db1=True)
    torch.cuda.synchronize()
    want = {**oracle.mlp_shard_fwd(X, A, x["B"], x["b1"], gelu),
            **oracle.mlp_shard_bwd(X, A, x["B"], x["dZ"], x["b1"], gelu)}
    got = {"H": host(H), "Y": host(Y), "Z": host(Z), "dA": host(dA), "dB": host(dB), "db1": host(db1), "dX": host(dX)}
    for k, v in got.items():
        assert np.isfinite(v).all(), k
    if label == "zeroA":
        assert np.abs(got["dX"]).max() == 0
        del got["dX"]
    errs = {k: rel_fro(v, want[k]) for k, v in got.items()}
    print("  rel-fro", {k: f"{e:.2e}" for k, e in errs.items()}, flush=True)
    assert all(e <= MLP_TOL for e in errs.values()), errs
