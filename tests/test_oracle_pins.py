"""Pins that tie the fp64 oracle to facts fixed outside itself (CPU only).

Each pin is chosen so that a plausible mistake in the oracle (a dropped term, a
wrong sign or index, a transposed operand) fails at least one of them; the
mutation tests at the end plant such mistakes in the oracle and check that.

Sources: Megatron-LM explainer (azimuth.plus) "core idea: slicing the
feed-forward network" and "the f and g operators"; Megatron-LM paper notes
(notes.yuuk.io) "MLP block split" and "vocab-embedding parallelism".
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy import special

import oracle
from oracle import ref
from tests.conftest import rel_fro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ----------------------------------------------------------------------------- GeLU
def test_gelu_textbook_cdf_values():
    """GeLU(x) = x Phi(x): textbook normal-CDF values (golden fixture)."""
    data = np.loadtxt(os.path.join(GOLDEN, "normal_cdf_textbook.txt"))
    x, phi = data[:, 0], data[:, 1]
    got = oracle.gelu(x, "erf")
    np.testing.assert_allclose(got, x * phi, rtol=1e-14, atol=1e-16)


@pytest.mark.parametrize("form", ["erf", "tanh"])
def test_gelu_closed_forms(form):
    """GeLU(0) = 0, GeLU'(0) = 1/2, GeLU(-x) = GeLU(x) - x (P7)."""
    x = np.linspace(-6, 6, 241)
    assert oracle.gelu(np.array([0.0]), form)[0] == 0.0
    assert oracle.gelu_grad(np.array([0.0]), form)[0] == 0.5
    np.testing.assert_allclose(oracle.gelu(-x, form), oracle.gelu(x, form) - x, rtol=0, atol=1e-14)


@pytest.mark.parametrize("form,approx", [("erf", "none"), ("tanh", "tanh")])
def test_gelu_matches_torch_fp64(form, approx):
    """Library special case (P8): torch's GeLU and its autograd derivative in fp64."""
    x = np.linspace(-8, 8, 1601)
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    ty = torch.nn.functional.gelu(tx, approximate=approx)
    ty.sum().backward()
    np.testing.assert_allclose(oracle.gelu(x, form), ty.detach().numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(oracle.gelu_grad(x, form), tx.grad.numpy(), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("form", ["erf", "tanh"])
def test_gelu_grad_finite_difference(form):
    x = np.linspace(-5, 5, 101)
    eps = 1e-6
    fd = (oracle.gelu(x + eps, form) - oracle.gelu(x - eps, form)) / (2 * eps)
    np.testing.assert_allclose(oracle.gelu_grad(x, form), fd, rtol=1e-7, atol=1e-9)


def test_gelu_erf_vs_tanh_gap():
    """The two GeLU forms differ by well under the 1e-2 tolerance (reading of the unnamed GeLU)."""
    x = np.linspace(-10, 10, 200001)
    gap = np.abs(oracle.gelu(x, "erf") - oracle.gelu(x, "tanh")).max()
    assert 1e-4 < gap < 1e-3


# ----------------------------------------------------------------------------- MLP identities
def _mlp_problem(rng, T=16, h=12, f=24, bias=True):
    X = _rand(rng, T, h)
    A = _rand(rng, h, f, scale=0.3)
    B = _rand(rng, f, h, scale=0.3)
    dZ = _rand(rng, T, h)
    b1 = _rand(rng, f, scale=0.3) if bias else None
    return X, A, B, dZ, b1


@pytest.mark.parametrize("t", [2, 3, 4])
@pytest.mark.parametrize("form", ["erf", "tanh"])
def test_column_shard_gelu_identity(rng, t, form):
    """P1 [EXPL core idea; NOTES MLP block split]: concat_r GeLU(X A_r) == GeLU(X A)."""
    X, A, B, dZ, b1 = _mlp_problem(rng, f=24)
    full = oracle.mlp_shard_fwd(X, A, B, b1, form)
    cuts = np.array_split(np.arange(A.shape[1]), t)
    Ys = [oracle.mlp_shard_fwd(X, A[:, c], B[c, :], b1[c], form)["Y"] for c in cuts]
    np.testing.assert_allclose(np.concatenate(Ys, axis=1), full["Y"], rtol=1e-15, atol=0)


@pytest.mark.parametrize("t", [2, 4, 5])
def test_row_parallel_partials_sum(rng, t):
    """P2 [EXPL core idea]: sum over ranks of Z_r = GeLU(X A_r) B_r equals GeLU(X A) B."""
    X, A, B, dZ, b1 = _mlp_problem(rng, f=40)
    full = oracle.mlp_shard_fwd(X, A, B, b1)["Z"]
    cuts = np.array_split(np.arange(A.shape[1]), t)
    s = sum(oracle.mlp_shard_fwd(X, A[:, c], B[c, :], b1[c])["Z"] for c in cuts)
    assert rel_fro(s, full) < 1e-13


def test_row_split_negative_control(rng):
    """P3 [EXPL core idea, the rejected first option]: splitting A by rows (X along h)
    and applying GeLU before the sum does NOT reproduce GeLU(X A); the identity
    checks above would fail for that split."""
    X, A, B, dZ, b1 = _mlp_problem(rng, T=64, h=64, f=256, bias=False)
    want = oracle.gelu(X @ A)
    for t in (2, 4):
        cuts = np.array_split(np.arange(X.shape[1]), t)
        wrong = sum(oracle.gelu(X[:, c] @ A[c, :]) for c in cuts)
        assert rel_fro(wrong, want) > 0.1


@pytest.mark.parametrize("form", ["erf", "tanh"])
@pytest.mark.parametrize("bias", [False, True])
def test_backward_finite_differences(rng, form, bias):
    """P4: the backward equals central finite differences of L = sum(dZ * Z_i)."""
    T, h, f = 3, 5, 7
    X, A, B, dZ, b1 = _mlp_problem(rng, T=T, h=h, f=f, bias=bias)
    g = oracle.mlp_shard_bwd(X, A, B, dZ, b1, form)

    def loss(X_, A_, B_, b1_):
        return float((dZ * oracle.mlp_shard_fwd(X_, A_, B_, b1_, form)["Z"]).sum())

    eps = 1e-6

    def fd(which):
        arrs = {"X": X, "A": A, "B": B, "b1": b1}
        base = arrs[which]
        out = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            p = {k: (v.copy() if v is not None else None) for k, v in arrs.items()}
            m = {k: (v.copy() if v is not None else None) for k, v in arrs.items()}
            p[which][idx] += eps
            m[which][idx] -= eps
            out[idx] = (loss(p["X"], p["A"], p["B"], p["b1"]) - loss(m["X"], m["A"], m["B"], m["b1"])) / (2 * eps)
        return out

    assert rel_fro(g["dX"], fd("X")) < 1e-7
    assert rel_fro(g["dA"], fd("A")) < 1e-7
    assert rel_fro(g["dB"], fd("B")) < 1e-7
    if bias:
        assert rel_fro(g["db1"], fd("b1")) < 1e-7


@pytest.mark.parametrize("t", [2, 4])
def test_backward_shard_identities(rng, t):
    """P5 [EXPL f and g operators]: sum_r dX_r = dX; [dA_1..dA_t] = dA; [dB_1;..;dB_t] = dB."""
    X, A, B, dZ, b1 = _mlp_problem(rng, T=20, h=16, f=32)
    full = oracle.mlp_shard_bwd(X, A, B, dZ, b1)
    cuts = np.array_split(np.arange(A.shape[1]), t)
    parts = [oracle.mlp_shard_bwd(X, A[:, c], B[c, :], dZ, b1[c]) for c in cuts]
    assert rel_fro(sum(p["dX"] for p in parts), full["dX"]) < 1e-13
    assert rel_fro(np.concatenate([p["dA"] for p in parts], axis=1), full["dA"]) < 1e-13
    assert rel_fro(np.concatenate([p["dB"] for p in parts], axis=0), full["dB"]) < 1e-13
    assert rel_fro(np.concatenate([p["db1"] for p in parts]), full["db1"]) < 1e-13


def test_mlp_closed_form_zero_A(rng):
    """P7: A = 0 (no bias) gives H = 0, Z = 0, dB = 0 and dH = dY / 2."""
    X, A, B, dZ, _ = _mlp_problem(rng, bias=False)
    A0 = np.zeros_like(A)
    f = oracle.mlp_shard_fwd(X, A0, B)
    g = oracle.mlp_shard_bwd(X, A0, B, dZ)
    assert not f["Z"].any() and not g["dB"].any()
    np.testing.assert_array_equal(g["dH"], 0.5 * (dZ @ B.T))


def test_sampled_matches_full(rng):
    X, A, B, dZ, b1 = _mlp_problem(rng, T=30, h=16, f=40)
    full_f = oracle.mlp_shard_fwd(X, A, B, b1)
    full_b = oracle.mlp_shard_bwd(X, A, B, dZ, b1)
    R, C = [0, 3, 29], [0, 7, 39]
    s = oracle.mlp_shard_sampled(X, A, B, dZ, R, C, b1)
    np.testing.assert_allclose(s["Z_rows"], full_f["Z"][R], rtol=1e-13)
    np.testing.assert_allclose(s["dX_rows"], full_b["dX"][R], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s["dA_cols"], full_b["dA"][:, C], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s["dB_cols"], full_b["dB"][C, :], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s["db1_cols"], full_b["db1"][C], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- scalar brute force
def _brute_mlp(X, A, B, dZ, b1, form):
    """P9: pure-Python loops with math.erf / math.tanh / math.exp and math.fsum."""
    T, h = len(X), len(X[0])
    f = len(A[0])

    def g(x):
        if form == "erf":
            return 0.5 * x * (1 + math.erf(x / math.sqrt(2)))
        return 0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))

    def gp(x):
        if form == "erf":
            return 0.5 * (1 + math.erf(x / math.sqrt(2))) + x * math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
        u = math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)
        return 0.5 * (1 + math.tanh(u)) + 0.5 * x * (1 - math.tanh(u) ** 2) * math.sqrt(2 / math.pi) * (
            1 + 3 * 0.044715 * x * x)

    H = [[math.fsum(X[t][k] * A[k][j] for k in range(h)) + b1[j] for j in range(f)] for t in range(T)]
    Y = [[g(H[t][j]) for j in range(f)] for t in range(T)]
    Z = [[math.fsum(Y[t][j] * B[j][c] for j in range(f)) for c in range(h)] for t in range(T)]
    dH = [[math.fsum(dZ[t][c] * B[j][c] for c in range(h)) * gp(H[t][j]) for j in range(f)] for t in range(T)]
    dA = [[math.fsum(X[t][k] * dH[t][j] for t in range(T)) for j in range(f)] for k in range(h)]
    dB = [[math.fsum(Y[t][j] * dZ[t][c] for t in range(T)) for c in range(h)] for j in range(f)]
    dX = [[math.fsum(dH[t][j] * A[k][j] for j in range(f)) for k in range(h)] for t in range(T)]
    db1 = [math.fsum(dH[t][j] for t in range(T)) for j in range(f)]
    return dict(H=H, Y=Y, Z=Z, dH=dH, dA=dA, dB=dB, dX=dX, db1=db1)


@pytest.mark.parametrize("form", ["erf", "tanh"])
def test_scalar_brute_force_mlp(rng, form):
    T, h, f = 3, 4, 8
    X, A, B, dZ, b1 = _mlp_problem(rng, T=T, h=h, f=f)
    want = _brute_mlp(X.tolist(), A.tolist(), B.tolist(), dZ.tolist(), b1.tolist(), form)
    fw = oracle.mlp_shard_fwd(X, A, B, b1, form)
    bw = oracle.mlp_shard_bwd(X, A, B, dZ, b1, form)
    for k in ("H", "Y", "Z"):
        np.testing.assert_allclose(fw[k], np.array(want[k]), rtol=1e-13, atol=1e-15)
    for k in ("dH", "dA", "dB", "dX", "db1"):
        np.testing.assert_allclose(bw[k], np.array(want[k]), rtol=1e-13, atol=1e-15)


def test_scalar_brute_force_ce(rng):
    T, h, v = 3, 4, 10
    X = _rand(rng, T, h)
    E = _rand(rng, h, v)
    y = np.array([0, 9, 4])
    L = [[math.fsum(X[t, k] * E[k, j] for k in range(h)) for j in range(v)] for t in range(T)]
    want = [math.log(math.fsum(math.exp(L[t][j]) for j in range(v))) - L[t][y[t]] for t in range(T)]
    np.testing.assert_allclose(oracle.full_vocab_ce(X, E, y), want, rtol=1e-14)
    for split in ([10], [4, 6], [3, 3, 4]):
        offs = np.cumsum([0] + split)
        parts = [oracle.vocab_ce_shard(X, E[:, offs[r]:offs[r + 1]], y, offs[r]) for r in range(len(split))]
        c = oracle.ce_combine([p["m"] for p in parts], [p["s"] for p in parts], [p["z"] for p in parts])
        np.testing.assert_allclose(c["loss"], want, rtol=1e-14)


# ----------------------------------------------------------------------------- CE identities
@pytest.mark.parametrize("split", [[96], [48, 48], [24, 24, 24, 24], [10, 50, 36], [1, 94, 1]])
def test_vocab_shard_ce_identity(rng, split):
    """P6 [NOTES vocab-embedding parallelism]: combining per-shard (m, s, z) over any
    vocab split equals the unsharded cross-entropy, including targets at shard edges."""
    T, h = 40, 16
    v = sum(split)
    X = _rand(rng, T, h)
    E = _rand(rng, h, v, scale=0.5)
    offs = np.cumsum([0] + split)
    edge = sorted({int(o) for o in offs[:-1]} | {int(o) - 1 for o in offs[1:]})
    y = rng.integers(0, v, size=T)
    y[:len(edge)] = edge[:T]
    parts = [oracle.vocab_ce_shard(X, E[:, offs[r]:offs[r + 1]], y, offs[r]) for r in range(len(split))]
    c = oracle.ce_combine([p["m"] for p in parts], [p["s"] for p in parts], [p["z"] for p in parts])
    full = oracle.full_vocab_ce(X, E, y)
    assert rel_fro(c["loss"], full) < 1e-13
    assert abs(c["mean"] - full.mean()) <= 1e-13 * abs(full.mean())
    # exactly one shard owns each target: z sums one nonzero with zeros
    owners = sum((np.asarray(p["z"]) != 0).astype(int) for p in parts)
    assert owners.max() <= 1


def test_ce_matches_torch_and_scipy(rng):
    """P8: t = 1 equals torch.nn.functional.cross_entropy (fp64) and scipy logsumexp."""
    T, h, v = 50, 24, 130
    X = _rand(rng, T, h)
    E = _rand(rng, h, v, scale=0.7)
    y = rng.integers(0, v, size=T)
    p = oracle.vocab_ce_shard(X, E, y, 0)
    c = oracle.ce_combine(p["m"], p["s"], p["z"])
    tl = torch.nn.functional.cross_entropy(torch.tensor(X @ E), torch.tensor(y), reduction="none").numpy()
    np.testing.assert_allclose(c["loss"], tl, rtol=1e-13)
    L = X @ E
    np.testing.assert_allclose(p["m"] + np.log(p["s"]), special.logsumexp(L, axis=1), rtol=1e-14)
    np.testing.assert_array_equal(p["m"], L.max(axis=1))


@pytest.mark.parametrize("zero", ["E", "X"])
def test_ce_closed_form_ln_v(rng, zero):
    """P7: all-zero logits give loss = ln v exactly, for any target and any split."""
    T, h, v = 9, 8, 64
    X = np.zeros((T, h)) if zero == "X" else _rand(rng, T, h)
    E = np.zeros((h, v)) if zero == "E" else _rand(rng, h, v)
    y = rng.integers(0, v, size=T)
    parts = [oracle.vocab_ce_shard(X, E[:, r * 16:(r + 1) * 16], y, r * 16) for r in range(4)]
    c = oracle.ce_combine([p["m"] for p in parts], [p["s"] for p in parts], [p["z"] for p in parts])
    np.testing.assert_allclose(c["loss"], math.log(v), rtol=1e-15)


def test_exchange_size_is_b_times_s():
    """[NOTES vocab-embedding parallelism]: the shard's output per quantity has b*s values."""
    b, s, v, unfused, fused = np.loadtxt(os.path.join(GOLDEN, "exchange_sizes.txt"), dtype=np.int64)
    assert b * s * v == unfused and b * s == fused
    T, h = int(b * s) // 64, 8       # a scaled-down token count with the same structure
    X = np.ones((T, h)); E = np.zeros((h, 32))
    p = oracle.vocab_ce_shard(X, E, np.zeros(T, dtype=np.int64), 0)
    assert all(np.asarray(p[k]).shape == (T,) for k in ("m", "s", "z"))


# ----------------------------------------------------------------------------- mutation checks
def _mutant_gelu_grad_no_pdf(x, form="erf"):
    return 0.5 * (1.0 + special.erf(x / math.sqrt(2.0)))  # drops the x*phi(x) term


def test_pins_catch_dropped_gelu_term(rng, monkeypatch):
    monkeypatch.setattr(ref, "gelu_grad", _mutant_gelu_grad_no_pdf)
    with pytest.raises(AssertionError):
        test_backward_finite_differences(rng, "erf", False)


def test_pins_catch_wrong_ce_sign(rng, monkeypatch):
    orig = ref.ce_combine

    def bad(m, s, z):
        out = orig(m, s, z)
        m2 = np.atleast_2d(m).max(axis=0)
        out["loss"] = out["loss"] - 2 * m2  # flips the sign of the max shift
        return out

    monkeypatch.setattr(oracle, "ce_combine", bad)
    with pytest.raises(AssertionError):
        test_ce_matches_torch_and_scipy(rng)


def test_pins_catch_transposed_weight_operand(rng, monkeypatch):
    orig = ref.mlp_shard_fwd

    def bad(X, A_i, B_i, b1_i=None, form="erf"):
        out = orig(X, A_i, B_i, b1_i, form)
        Xf = ref._f64(X)
        Af = ref._f64(A_i)
        H = Xf @ Af
        if b1_i is not None:
            H = H + ref._f64(b1_i)[None, :]
        out["Z"] = ref.gelu(H, form) @ ref._f64(B_i)[::-1, :]  # row order of B_i reversed
        return out

    monkeypatch.setattr(oracle, "mlp_shard_fwd", bad)
    with pytest.raises(AssertionError):
        test_scalar_brute_force_mlp(rng, "erf")


def test_pins_catch_wrong_target_offset(rng, monkeypatch):
    orig = ref.vocab_ce_shard

    def bad(X, E_i, targets, vocab_start, rows=None, block=512):
        return orig(X, E_i, targets, vocab_start + 1, rows, block)  # off-by-one ownership

    monkeypatch.setattr(oracle, "vocab_ce_shard", bad)
    with pytest.raises(AssertionError):
        test_vocab_shard_ce_identity(rng, [48, 48])


# ----------------------------------------------------------------------------- input widening
def _bf16_by_definition(u: int) -> float:
    """bf16 bit pattern -> value from the format's definition (1 sign bit, 8
    exponent bits with bias 127, 7 fraction bits; subnormals, infinities, NaN)."""
    sign = -1.0 if (u >> 15) & 1 else 1.0
    e = (u >> 7) & 0xFF
    f = u & 0x7F
    if e == 0xFF:
        return math.nan if f else sign * math.inf
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


def test_bf16_widening_every_bit_pattern():
    """bf16_to_f64 on all 65536 patterns equals the format's definition and
    torch's bfloat16 -> float64 conversion (NaN patterns stay NaN)."""
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f64(u)
    assert got.dtype == np.float64 and got.shape == (1 << 16,)
    want = np.array([_bf16_by_definition(int(x)) for x in u], dtype=np.float64)
    nan = np.isnan(want)
    assert nan.sum() == 2 * 127  # both signs, every nonzero fraction
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0 and math.copysign(1.0, got[0]) == 1.0
    tv = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(tv), nan)
    np.testing.assert_array_equal(got[~nan], tv[~nan])


def test_oracle_entry_points_widen_bf16_inputs(rng):
    """The oracle's functions take raw bf16 patterns (uint16) and give exactly
    what they give on the same values already widened to float64."""
    T, h, f, v = 6, 8, 16, 24
    bits = lambda *s: (rng.integers(0, 1 << 16, size=s, dtype=np.uint32) & 0x3FFF | 0x3000).astype(np.uint16)
    X, A, B, E, dZ = bits(T, h), bits(h, f), bits(f, h), bits(h, v), bits(T, h)
    w = lambda a: torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    y = rng.integers(0, v, size=T)
    fb, fw = oracle.mlp_shard_fwd(X, A, B), oracle.mlp_shard_fwd(w(X), w(A), w(B))
    bb, bw = oracle.mlp_shard_bwd(X, A, B, dZ), oracle.mlp_shard_bwd(w(X), w(A), w(B), w(dZ))
    cb, cw = oracle.vocab_ce_shard(X, E, y, 0), oracle.vocab_ce_shard(w(X), w(E), y, 0)
    for got, want in [(fb, fw), (bb, bw), (cb, cw)]:
        for k in want:
            np.testing.assert_array_equal(got[k], want[k])


# ----------------------------------------------------------------------------- CE over several token blocks
@pytest.mark.parametrize("T", [1100, 1536])
def test_ce_across_token_blocks(rng, T):
    """The CE oracle walks tokens 512 at a time (memory only).  At T past two
    block edges: the combined vocab shards and the unsharded CE equal torch's
    cross_entropy (fp64) on every token, and a permuted row subset gives the
    same values as the full evaluation."""
    h, split = 8, [40, 24, 33]
    v = sum(split)
    X = _rand(rng, T, h)
    E = _rand(rng, h, v, scale=0.8)
    y = rng.integers(0, v, size=T)
    offs = np.cumsum([0] + split)
    parts = [oracle.vocab_ce_shard(X, E[:, offs[r]:offs[r + 1]], y, int(offs[r])) for r in range(len(split))]
    c = oracle.ce_combine([p["m"] for p in parts], [p["s"] for p in parts], [p["z"] for p in parts])
    tl = torch.nn.functional.cross_entropy(torch.tensor(X @ E), torch.tensor(y), reduction="none").numpy()
    np.testing.assert_allclose(c["loss"], tl, rtol=1e-13)
    np.testing.assert_allclose(oracle.full_vocab_ce(X, E, y), tl, rtol=1e-13)
    assert abs(c["mean"] - math.fsum(tl.tolist()) / T) <= 1e-13 * abs(tl.mean())
    R = rng.permutation(T)[: T - 3]
    np.testing.assert_allclose(oracle.full_vocab_ce(X, E, y, rows=R), tl[R], rtol=1e-13)
    sub = oracle.vocab_ce_shard(X, E, y, 0, rows=R)
    np.testing.assert_allclose(sub["m"] + np.log(sub["s"]) - sub["z"], tl[R], rtol=1e-13)


def test_pins_catch_bf16_shift_of_15(monkeypatch):
    def bad(u):
        u32 = np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 15
        return u32.view(np.float32).astype(np.float64)

    monkeypatch.setattr(oracle, "bf16_to_f64", bad)
    with pytest.raises(AssertionError):
        test_bf16_widening_every_bit_pattern()


def test_pins_catch_token_block_offset(rng, monkeypatch):
    """A block walk whose second and later blocks start one token late."""
    def bad_full(X, E, targets, rows=None, block=512):
        X, E = ref._f64(X), ref._f64(E)
        targets = np.asarray(targets, dtype=np.int64)
        R = np.arange(X.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
        out = np.empty(len(R))
        for b0 in range(0, len(R), block):
            s0 = b0 + (1 if b0 else 0)
            rb = R[s0:s0 + block]
            L = X[rb] @ E
            val = special.logsumexp(L, axis=1) - L[np.arange(len(rb)), targets[rb]]
            out[b0:b0 + len(val)] = val
        return out

    monkeypatch.setattr(oracle, "full_vocab_ce", bad_full)
    with pytest.raises(AssertionError):
        test_ce_across_token_blocks(rng, 1100)


def test_pins_catch_shard_block_offset(rng, monkeypatch):
    """The same planted mistake in the shard partials' block walk."""
    orig = ref.vocab_ce_shard

    def bad(X, E_i, targets, vocab_start, rows=None, block=512):
        n = np.asarray(X).shape[0]
        R = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
        R = np.concatenate([R[:block], R[block + 1:], R[-1:]])  # later blocks one token late
        return orig(X, E_i, targets, vocab_start, rows=R, block=block)

    monkeypatch.setattr(oracle, "vocab_ce_shard", bad)
    with pytest.raises(AssertionError):
        test_ce_across_token_blocks(rng, 1100)


def test_pins_catch_bf16_shift_inside_entry_points(rng, monkeypatch):
    def bad(u):
        u32 = np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 15
        return u32.view(np.float32).astype(np.float64)

    monkeypatch.setattr(ref, "bf16_to_f64", bad)
    with pytest.raises(AssertionError):
        test_oracle_entry_points_widen_bf16_inputs(rng)
