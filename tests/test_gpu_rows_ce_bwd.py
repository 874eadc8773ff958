"""GPU parity of the vocab-parallel cross-entropy backward against the fp64 oracle.

Both sides take the same inputs: seeded bf16 X, E_i, targets, per-token weights,
and the forward partials (m, s) of every vocab shard, which the oracle computes
in fp64 and which are rounded to fp32 for both sides.  Tolerance: relative
Frobenius error <= 1e-2 on dX_i and dE_i, the bar for bf16 gradients.

Sizes: full comparisons on shapes that span several 256-wide tiles with ragged
tails, single-token and sub-tile shapes; at the four large workloads' full
sizes, sampled token rows of dX_i and vocab columns of dE_i (tile edges always
included), each of which the oracle evaluates on its own.
"""
import hashlib

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_mlp_amd import inputs
from tests.conftest import rel_fro

pytestmark = pytest.mark.gpu

TOL = 1e-2


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


def f32(x) -> np.ndarray:
    """The oracle's fp64 partials as the fp32 values both sides receive."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def shard_partials(X, shards, targets, v_i):
    """Forward partials (m, s) of every vocab shard, by the oracle, rank order."""
    m, s = [], []
    for r, E in enumerate(shards):
        o = oracle.vocab_ce_shard(X, E, targets, r * v_i)
        m.append(o["m"]); s.append(o["s"])
    return f32(m), f32(s)


def weights(T, seed, zero_every=0):
    w = np.random.Generator(np.random.PCG64(seed)).uniform(0.25, 1.75, size=T).astype(np.float32)
    if zero_every:
        w[::zero_every] = 0.0  # masked tokens
    return w


def run_bwd(ms, X, E, targets, m, s, rank, v_i, dloss=None, grad_scale=None, workspace=None):
    dX, dE = ms.vocab_ce_shard_bwd(dev(X) if isinstance(X, np.ndarray) else X, dev(E),
                                   torch.from_numpy(targets).cuda(), torch.from_numpy(m).cuda(),
                                   torch.from_numpy(s).cuda(), rank * v_i,
                                   dloss=None if dloss is None else torch.from_numpy(dloss).cuda(),
                                   grad_scale=grad_scale, workspace=workspace)
    torch.cuda.synchronize()
    return dX, dE


# ----------------------------------------------------------------------------- full comparisons
@pytest.mark.parametrize("T,h,v,t,rank", [(64, 64, 512, 1, 0), (600, 392, 1000, 2, 1), (300, 136, 520, 3, 2),
                                          (37, 72, 40, 2, 0), (1, 8, 8, 1, 0)])
def test_ce_bwd_full(ms, T, h, v, t, rank):
    """All outputs in full: ragged M/N tails, a K tail (h % 32 != 0), several tiles,
    a shard that is not the first (targets owned by other ranks), and tiny shapes.
    Per-token weights with masked (zero-weight) tokens."""
    print(f"case ce_bwd full T={T} h={h} v_i={v} t={t} rank={rank}", flush=True)
    d = inputs.make_inputs(T, h, 8, v, t=t, rank=rank, v_global=t * v)
    shards = [inputs.make_inputs(T, h, 8, v, t=t, rank=r, v_global=t * v)["E"] for r in range(t)]
    assert np.array_equal(shards[rank], d["E"])
    m, s = shard_partials(d["X"], shards, d["targets"], v)
    w = weights(T, 7, zero_every=5)
    dX, dE = run_bwd(ms, d["X"], d["E"], d["targets"], m, s, rank, v, dloss=w, grad_scale=1.0 / T)
    o = oracle.vocab_ce_shard_bwd(d["X"], d["E"], d["targets"], rank * v, m, s, w.astype(np.float64) / T)
    errs = {"dX": rel_fro(host(dX), o["dX"]), "dE": rel_fro(host(dE), o["dE"])}
    print("  rel-fro", {k: f"{e:.2e}" for k, e in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= TOL, (k, e)
    # masked tokens get exactly zero input gradient
    assert not host(dX)[::5].any()


def test_ce_bwd_target_edges(ms):
    """Targets on this shard's first and last columns, just outside it, and at the
    256-column tile boundary; the mean's default weight 1/T."""
    T, h, v, t, rank = 300, 136, 520, 3, 1
    print(f"case ce_bwd edges T={T} h={h} v_i={v}", flush=True)
    d = inputs.make_inputs(T, h, 8, v, t=t, rank=rank, v_global=t * v)
    start = rank * v
    tg = d["targets"].copy()
    tg[:6] = [start, start + v - 1, start - 1, start + v, start + 255, start + 256]
    shards = [inputs.make_inputs(T, h, 8, v, t=t, rank=r, v_global=t * v)["E"] for r in range(t)]
    m, s = shard_partials(d["X"], shards, tg, v)
    dX, dE = run_bwd(ms, d["X"], d["E"], tg, m, s, rank, v)
    o = oracle.vocab_ce_shard_bwd(d["X"], d["E"], tg, start, m, s, np.full(T, 1.0 / T))
    assert rel_fro(host(dX), o["dX"]) <= TOL
    assert rel_fro(host(dE), o["dE"]) <= TOL


# ----------------------------------------------------------------------------- multi-rank emulation
@pytest.mark.parametrize("t", [2, 4])
def test_ce_bwd_tensor_parallel_emulation(ms, t):
    """All t vocab shards end to end on one GPU (forward partials from the GPU,
    backward on the GPU): the sum of the dX_r partials (what the exchange would
    all-reduce) and the dE_r slices side by side match the unsharded backward."""
    T, h, v = 512, 256, 2048
    print(f"case ce_bwd emulation t={t}", flush=True)
    d = inputs.make_inputs(T, h, 8, v)
    X, tg = dev(d["X"]), torch.from_numpy(d["targets"]).cuda()
    vs = v // t
    Es = [dev(np.ascontiguousarray(d["E"][:, r * vs:(r + 1) * vs])) for r in range(t)]
    parts = [ms.vocab_ce_shard_fwd(X, Es[r], tg, r * vs) for r in range(t)]
    m = torch.stack([p[0] for p in parts])
    s = torch.stack([p[1] for p in parts])
    dXs, dEs = 0, []
    for r in range(t):
        dX, dE = ms.vocab_ce_shard_bwd(X, Es[r], tg, m, s, r * vs)
        dXs = dXs + host(dX)
        dEs.append(host(dE))
    torch.cuda.synchronize()
    om, os_ = shard_partials(d["X"], [d["E"]], d["targets"], v)
    o = oracle.vocab_ce_shard_bwd(d["X"], d["E"], d["targets"], 0, om, os_, np.full(T, 1.0 / T))
    assert rel_fro(dXs, o["dX"]) <= TOL
    assert rel_fro(np.hstack(dEs), o["dE"]) <= TOL


# ----------------------------------------------------------------------------- full-size sampled
BIG = ["gpt2_1p5b", "gpt_8p3b_t8", "bert_3p9b_t4", "bloom_176b_t4"]


@pytest.mark.parametrize("name", BIG)
def test_ce_bwd_full_size_sampled(ms, name):
    """Shard 0 of each workload at its real shape, in the launch configuration a
    timed run uses: dX_i on 128 sampled tokens, dE_i on 128 sampled vocab columns."""
    c = inputs.CONFIGS[name]
    print(f"case ce_bwd {name} T={c.T} h={c.h} v_i={c.v_i} t={c.t}: oracle partials", flush=True)
    base = inputs.make_config_inputs(c, want=("X", "targets"))
    shards = []
    m, s = [], []
    for r in range(c.t):
        E = inputs.make_config_inputs(c, rank=r, want=("E",))["E"]
        o = oracle.vocab_ce_shard(base["X"], E, base["targets"], r * c.v_i)
        m.append(o["m"]); s.append(o["s"])
        shards.append(E if r == 0 else None)
        print(f"  shard {r} partials done", flush=True)
    m, s = f32(m), f32(s)
    E0 = shards[0]
    rows = inputs.sample_indices(c.T, 128, 21, [0, 255, 256, c.T - 1])
    cols = inputs.sample_indices(c.v_i, 128, 22, [0, 255, 256, c.v_i - 1])
    print("  gpu backward", flush=True)
    dX, dE = run_bwd(ms, base["X"], E0, base["targets"], m, s, 0, c.v_i)
    print("  oracle samples", flush=True)
    o = oracle.vocab_ce_shard_bwd(base["X"], E0, base["targets"], 0, m, s, np.full(c.T, 1.0 / c.T),
                                  rows=rows, cols=cols)
    R = torch.from_numpy(rows).cuda()
    C = torch.from_numpy(cols).cuda()
    errs = {"dX": rel_fro(host(dX[R]), o["dX_rows"]), "dE": rel_fro(host(dE[:, C]), o["dE_cols"])}
    print(f"  {name}", {k: f"{e:.2e}" for k, e in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= TOL, (k, e)


# ----------------------------------------------------------------------------- determinism
def test_ce_bwd_bitwise_determinism(ms):
    """Repeated calls give identical output bytes, with a workspace dirtied differently each time."""
    T, h, v = 4100, 392, 1000
    d = inputs.make_inputs(T, h, 8, v, t=2, rank=1, v_global=2 * v)
    shards = [inputs.make_inputs(T, h, 8, v, t=2, rank=r, v_global=2 * v)["E"] for r in range(2)]
    m, s = shard_partials(d["X"], shards, d["targets"], v)
    X = dev(d["X"])
    ref = None
    for it in range(10):
        ws = torch.full((ms.vocab_ce_bwd_workspace_bytes(T, h, v),), it, dtype=torch.uint8, device="cuda")
        dX, dE = run_bwd(ms, X, d["E"], d["targets"], m, s, 1, v, workspace=ws)
        hsh = hashlib.sha256()
        for x in (dX, dE):
            hsh.update(x.contiguous().view(torch.uint8).cpu().numpy().tobytes())
        ref = ref or hsh.hexdigest()
        assert hsh.hexdigest() == ref, it


def test_ce_degenerate_and_extreme_logits(ms):
    """E = 0 (every logit 0: m = 0, s = v_i and z = 0 exactly, dX_i = 0) and logits
    64 times the workloads' scale (the shard max keeps every exponential finite)."""
    T, h, v = 300, 128, 520
    print(f"case ce degenerate T={T} h={h} v={v}", flush=True)
    d = inputs.make_inputs(T, h, 8, v)
    tg = torch.from_numpy(d["targets"]).cuda()
    E0 = np.zeros_like(d["E"])
    m, s, z = ms.vocab_ce_shard_fwd(dev(d["X"]), dev(E0), tg, 0)
    torch.cuda.synchronize()
    assert (host(m) == 0).all() and (host(s) == v).all() and (host(z) == 0).all()
    dX, dE = run_bwd(ms, d["X"], E0, d["targets"], f32(host(m)[None]), f32(host(s)[None]), 0, v)
    ob = oracle.vocab_ce_shard_bwd(d["X"], E0, d["targets"], 0, host(m)[None], host(s)[None], 1.0 / T)
    assert np.abs(host(dX)).max() == 0
    assert rel_fro(host(dE), ob["dE"]) <= TOL
    Xb = inputs.round_to_bf16_bits(inputs.bf16_bits_to_f32(d["X"]) * np.float32(64.0))
    m, s, z = ms.vocab_ce_shard_fwd(dev(Xb), dev(d["E"]), tg, 0)
    torch.cuda.synchronize()
    o = oracle.vocab_ce_shard(Xb, d["E"], d["targets"], 0)
    assert np.abs(host(m) - o["m"]).max() <= 1e-4 * np.abs(o["m"]).max()
    assert np.abs(host(s) / o["s"] - 1).max() <= 1e-4
    dX, dE = run_bwd(ms, Xb, d["E"], d["targets"], f32(host(m)[None]), f32(host(s)[None]), 0, v)
    ob = oracle.vocab_ce_shard_bwd(Xb, d["E"], d["targets"], 0, host(m)[None], host(s)[None], 1.0 / T)
    assert rel_fro(host(dX), ob["dX"]) <= TOL
    assert rel_fro(host(dE), ob["dE"]) <= TOL
