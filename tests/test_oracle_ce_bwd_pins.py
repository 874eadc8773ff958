"""Pins for the oracle's vocab-parallel cross-entropy backward (CPU only).

The pages fuse the output GEMM with the cross-entropy on vocab shards (Megatron-LM
paper notes, notes.yuuk.io, "vocab-embedding parallelism") and give only the
forward.  The backward is the textbook softmax cross-entropy derivative carried
through the logits GEMM.  The pins tie it to facts outside the oracle:
torch autograd in fp64, finite differences of the already-pinned forward loss,
the shard identities, closed forms, the zero-row-sum invariant, and pure-Python
loops.  The mutation tests at the end plant mistakes in the oracle and check
that some pin fails.
"""
import math

import numpy as np
import pytest
import torch
from scipy import special

import oracle
from oracle import ref
from tests.conftest import rel_fro


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _shards(X, E, y, split):
    """Forward partials of every vocab shard, as the exchange would gather them."""
    offs = np.cumsum([0] + list(split))
    parts = [oracle.vocab_ce_shard(X, E[:, offs[r]:offs[r + 1]], y, offs[r]) for r in range(len(split))]
    m = np.stack([p["m"] for p in parts])
    s = np.stack([p["s"] for p in parts])
    return offs, m, s


def _bwd_full(X, E, y, coef):
    """Unsharded backward (one shard holding the whole vocabulary)."""
    _, m, s = _shards(X, E, y, [E.shape[1]])
    return oracle.vocab_ce_shard_bwd(X, E, y, 0, m, s, coef)


def test_row_stats_are_logsumexp(rng):
    """Combined (M, S) over any split gives M + ln S = scipy logsumexp of the full row."""
    T, h, v = 30, 12, 90
    X = _rand(rng, T, h)
    E = _rand(rng, h, v)
    y = rng.integers(0, v, size=T)
    for split in ([90], [45, 45], [7, 80, 3]):
        _, m, s = _shards(X, E, y, split)
        st = oracle.ce_row_stats(m, s)
        np.testing.assert_allclose(st["M"] + np.log(st["S"]), special.logsumexp(X @ E, axis=1), rtol=1e-14)
        np.testing.assert_array_equal(st["M"], (X @ E).max(axis=1))


@pytest.mark.parametrize("weights", ["mean", "per_token"])
def test_ce_bwd_matches_torch_autograd(rng, weights):
    """t = 1 equals torch autograd of sum_t coef_t * cross_entropy_t in fp64."""
    T, h, v = 50, 24, 130
    X = _rand(rng, T, h)
    E = _rand(rng, h, v, scale=0.7)
    y = rng.integers(0, v, size=T)
    coef = np.full(T, 1.0 / T) if weights == "mean" else rng.uniform(-1.0, 2.0, size=T)
    Xt = torch.tensor(X, requires_grad=True)
    Et = torch.tensor(E, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(Xt @ Et, torch.tensor(y), reduction="none")
    (loss * torch.tensor(coef)).sum().backward()
    g = _bwd_full(X, E, y, coef)
    np.testing.assert_allclose(g["dX"], Xt.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(g["dE"], Et.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_ce_bwd_finite_differences(rng):
    """Central differences of sum_t coef_t * loss_t, with the loss from the unsharded
    forward (itself pinned against torch and scipy)."""
    T, h, v = 3, 4, 10
    X = _rand(rng, T, h)
    E = _rand(rng, h, v)
    y = np.array([0, 9, 4])
    coef = np.array([0.5, -1.25, 2.0])

    def obj(Xv, Ev):
        return float(np.dot(coef, oracle.full_vocab_ce(Xv, Ev, y)))

    eps = 1e-6
    fdX = np.zeros_like(X)
    for idx in np.ndindex(*X.shape):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += eps
        Xm[idx] -= eps
        fdX[idx] = (obj(Xp, E) - obj(Xm, E)) / (2 * eps)
    fdE = np.zeros_like(E)
    for idx in np.ndindex(*E.shape):
        Ep, Em = E.copy(), E.copy()
        Ep[idx] += eps
        Em[idx] -= eps
        fdE[idx] = (obj(X, Ep) - obj(X, Em)) / (2 * eps)
    g = _bwd_full(X, E, y, coef)
    assert rel_fro(g["dX"], fdX) < 1e-7
    assert rel_fro(g["dE"], fdE) < 1e-7


@pytest.mark.parametrize("split", [[48, 48], [24, 24, 24, 24], [10, 50, 36], [1, 94, 1]])
def test_ce_bwd_shard_identity(rng, split):
    """Sharded backward: the ranks' dX partials sum to the unsharded dX, and the
    ranks' dE slices side by side are the unsharded dE; targets sit on shard edges."""
    T, h = 40, 16
    v = sum(split)
    X = _rand(rng, T, h)
    E = _rand(rng, h, v, scale=0.5)
    y = rng.integers(0, v, size=T)
    offs = np.cumsum([0] + split)
    edge = sorted({int(o) for o in offs[:-1]} | {int(o) - 1 for o in offs[1:]})
    y[:len(edge)] = edge[:T]
    coef = rng.uniform(0.1, 1.0, size=T)
    full = _bwd_full(X, E, y, coef)
    offs, m, s = _shards(X, E, y, split)
    parts = [oracle.vocab_ce_shard_bwd(X, E[:, offs[r]:offs[r + 1]], y, offs[r], m, s, coef)
             for r in range(len(split))]
    assert rel_fro(sum(p["dX"] for p in parts), full["dX"]) < 1e-13
    assert rel_fro(np.hstack([p["dE"] for p in parts]), full["dE"]) < 1e-13
    assert rel_fro(np.hstack([p["dL"] for p in parts]), full["dL"]) < 1e-13


def test_ce_bwd_invariants_and_closed_forms(rng):
    """Softmax minus one-hot sums to zero over the vocabulary, so dL's rows and dE's
    rows sum to zero; with E = 0 the softmax is uniform (1/v) and dX = 0 while
    dE[:, j] = sum_t coef_t X[t, :] (1/v - [y_t = j])."""
    T, h, v = 20, 8, 64
    X = _rand(rng, T, h)
    y = rng.integers(0, v, size=T)
    coef = rng.uniform(0.2, 1.0, size=T)
    g = _bwd_full(X, _rand(rng, h, v), y, coef)
    assert np.abs(g["dL"].sum(axis=1)).max() < 1e-15
    assert np.abs(g["dE"].sum(axis=1)).max() < 1e-14 * np.abs(g["dE"]).max()
    # the target column is the only negative entry of each row (softmax <= 1)
    assert (g["dL"] < 0).sum() == T and all(g["dL"][t, y[t]] < 0 for t in range(T))
    g0 = _bwd_full(X, np.zeros((h, v)), y, coef)
    assert np.all(g0["dX"] == 0.0)
    want = np.zeros((h, v))
    for t in range(T):
        want += coef[t] * np.outer(X[t], np.full(v, 1.0 / v) - (np.arange(v) == y[t]))
    np.testing.assert_allclose(g0["dE"], want, rtol=1e-13, atol=1e-16)


def test_ce_bwd_sampled_matches_full(rng):
    """Sampled rows of dX and columns of dE equal the full evaluation."""
    T, h, v = 70, 16, 200
    X = _rand(rng, T, h)
    E = _rand(rng, h, v, scale=0.5)
    y = rng.integers(0, v, size=T)
    coef = np.full(T, 1.0 / T)
    offs, m, s = _shards(X, E, y, [120, 80])
    full = oracle.vocab_ce_shard_bwd(X, E[:, 120:], y, 120, m, s, coef)
    R = [0, 5, 69, 33]
    C = [0, 1, 79, 40, 63, 64]
    smp = oracle.vocab_ce_shard_bwd(X, E[:, 120:], y, 120, m, s, coef, rows=R, cols=C)
    np.testing.assert_allclose(smp["dX_rows"], full["dX"][R], rtol=1e-14, atol=1e-18)
    np.testing.assert_allclose(smp["dE_cols"], full["dE"][:, C], rtol=1e-14, atol=1e-18)
    np.testing.assert_allclose(smp["dL_rows"], full["dL"][R], rtol=1e-14, atol=1e-20)


def test_scalar_brute_force_ce_bwd(rng):
    """Pure-Python loops (math.exp, math.fsum) against the numpy oracle on two shards."""
    T, h, v = 3, 4, 10
    X = _rand(rng, T, h)
    E = _rand(rng, h, v)
    y = np.array([0, 9, 4])
    coef = [0.3, 1.1, -0.7]
    L = [[math.fsum(X[t, k] * E[k, j] for k in range(h)) for j in range(v)] for t in range(T)]
    dL = []
    for t in range(T):
        mx = max(L[t])
        den = math.fsum(math.exp(L[t][j] - mx) for j in range(v))
        dL.append([coef[t] * (math.exp(L[t][j] - mx) / den - (1.0 if j == y[t] else 0.0)) for j in range(v)])
    dX = [[math.fsum(dL[t][j] * E[k, j] for j in range(v)) for k in range(h)] for t in range(T)]
    dE = [[math.fsum(X[t, k] * dL[t][j] for t in range(T)) for j in range(v)] for k in range(h)]
    offs, m, s = _shards(X, E, y, [4, 6])
    parts = [oracle.vocab_ce_shard_bwd(X, E[:, offs[r]:offs[r + 1]], y, offs[r], m, s, coef) for r in range(2)]
    np.testing.assert_allclose(parts[0]["dX"] + parts[1]["dX"], dX, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(np.hstack([parts[0]["dE"], parts[1]["dE"]]), dE, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------- mutation checks
def test_pins_catch_missing_one_hot(rng, monkeypatch):
    def bad(L, M, S, coef, targets, vocab_start, cols):
        return coef[:, None] * (np.exp(L - M[:, None]) / S[:, None])  # drops the target term

    monkeypatch.setattr(ref, "_ce_grad_block", bad)
    with pytest.raises(AssertionError):
        test_ce_bwd_matches_torch_autograd(rng, "mean")


def test_pins_catch_local_softmax(rng, monkeypatch):
    orig = ref.ce_row_stats

    def bad(m, s):
        out = orig(np.atleast_2d(m)[-1:], np.atleast_2d(s)[-1:])  # last shard's statistics only
        return out

    monkeypatch.setattr(ref, "ce_row_stats", bad)
    with pytest.raises(AssertionError):
        test_ce_bwd_shard_identity(rng, [48, 48])


def test_pins_catch_shifted_target_column(rng, monkeypatch):
    orig = ref._ce_grad_block

    def bad(L, M, S, coef, targets, vocab_start, cols):
        return orig(L, M, S, coef, targets, vocab_start - 1, cols)  # one-hot one column late

    monkeypatch.setattr(ref, "_ce_grad_block", bad)
    with pytest.raises(AssertionError):
        test_scalar_brute_force_ce_bwd(rng)


def test_pins_catch_transposed_gemm_operand(rng, monkeypatch):
    orig = ref.vocab_ce_shard_bwd

    def bad(X, E_i, targets, vocab_start, m, s, coef, rows=None, cols=None):
        out = orig(X, E_i, targets, vocab_start, m, s, coef, rows, cols)
        if "dE" in out:
            out["dE"] = ref._f64(X)[::-1].T @ out["dL"]  # token order of X reversed
        return out

    monkeypatch.setattr(oracle, "vocab_ce_shard_bwd", bad)
    with pytest.raises(AssertionError):
        test_ce_bwd_matches_torch_autograd(rng, "per_token")
