"""Pins for the oracle's self-attention shard (CPU only).

The pages split attention by heads: Q, K, V projections column-parallel per
head, the output projection row-parallel (Megatron-LM explainer, azimuth.plus,
"attention"; Megatron-LM paper notes, notes.yuuk.io, "self-attention block
split").  The per-head computation is the textbook scaled dot-product
attention.  The pins tie the oracle to facts outside itself: torch's own
scaled_dot_product_attention and autograd in fp64, finite differences, the
head-shard identities (with a negative control), closed forms of uniform
attention, and pure-Python loops.  The mutation tests plant mistakes in the
oracle and check that some pin fails.
"""
import math

import numpy as np
import pytest
import torch
from scipy import special

from oracle import attn
from tests.conftest import rel_fro


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _problem(rng, b=2, s=5, nh=4, d=3, scale_w=0.5):
    h = nh * d
    X = _rand(rng, b * s, h)
    Wq, Wk, Wv, Wo = (_rand(rng, h, h, scale=scale_w) for _ in range(4))
    dZ = _rand(rng, b * s, h)
    return X, Wq, Wk, Wv, Wo, dZ


def _rank_weights(Wq, Wk, Wv, Wo, t, r, nh, d):
    """Rank r's shard: columns of its nh/t heads from each projection, the matching rows of W_O."""
    n = nh // t
    c = slice(r * n * d, (r + 1) * n * d)
    return np.hstack([Wq[:, c], Wk[:, c], Wv[:, c]]), Wo[c, :], n


def _torch_shard(X, Wqkv, Wo, dZ, n, d, b, s, causal):
    """The same shard through torch (fp64, CPU): scaled_dot_product_attention and autograd."""
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(Wqkv, requires_grad=True)
    Ot = torch.tensor(Wo, requires_grad=True)
    qkv = Xt @ Wt
    nd = n * d

    def heads(x):  # [b*s, n*d] -> [b, n, s, d]
        return x.reshape(b, s, n, d).permute(0, 2, 1, 3)

    o = torch.nn.functional.scaled_dot_product_attention(heads(qkv[:, :nd]), heads(qkv[:, nd:2 * nd]),
                                                         heads(qkv[:, 2 * nd:]), is_causal=causal)
    O = o.permute(0, 2, 1, 3).reshape(b * s, nd)
    Z = O @ Ot
    (Z * torch.tensor(dZ)).sum().backward()
    return {"O": O.detach().numpy(), "Z": Z.detach().numpy(), "dX": Xt.grad.numpy(), "dWqkv": Wt.grad.numpy(),
            "dWo": Ot.grad.numpy()}


@pytest.mark.parametrize("causal", [True, False])
def test_attn_matches_torch_sdpa_and_autograd(rng, causal):
    """t = 1: forward and every gradient equal torch's fp64 attention and autograd."""
    b, s, nh, d = 2, 7, 4, 3
    X, Wq, Wk, Wv, Wo, dZ = _problem(rng, b, s, nh, d)
    Wqkv = np.hstack([Wq, Wk, Wv])
    want = _torch_shard(X, Wqkv, Wo, dZ, nh, d, b, s, causal)
    fw = attn.attn_shard_fwd(X, Wqkv, Wo, nh, d, b, s, causal)
    bw = attn.attn_shard_bwd(X, Wqkv, Wo, dZ, nh, d, b, s, causal)
    np.testing.assert_allclose(fw["O"], want["O"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fw["Z"], want["Z"], rtol=1e-12, atol=1e-14)
    for k in ("dX", "dWqkv", "dWo"):
        np.testing.assert_allclose(bw[k], want[k], rtol=1e-11, atol=1e-13)


def test_attn_lse_is_logsumexp(rng):
    """The saved per-row statistic is scipy's logsumexp of the scaled, masked scores."""
    b, s, nh, d = 1, 6, 2, 4
    X, Wq, Wk, Wv, Wo, _ = _problem(rng, b, s, nh, d)
    fw = attn.attn_shard_fwd(X, np.hstack([Wq, Wk, Wv]), Wo, nh, d, b, s, True)
    Q, K = X @ Wq, X @ Wk
    for j in range(nh):
        S = Q[:, j * d:(j + 1) * d] @ K[:, j * d:(j + 1) * d].T / math.sqrt(d)
        S[np.triu_indices(s, 1)] = -np.inf
        np.testing.assert_allclose(fw["lse"][j], special.logsumexp(S, axis=1), rtol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("t", [2, 4])
def test_attn_head_shard_identities(rng, t, causal):
    """Splitting the heads over t ranks: the O_r side by side are the unsharded O,
    the Z_r partials sum to the unsharded Z, the dX_r partials sum to dX, and each
    rank's weight gradients are the matching columns / rows of the unsharded ones."""
    b, s, nh, d = 2, 6, 8, 3
    X, Wq, Wk, Wv, Wo, dZ = _problem(rng, b, s, nh, d)
    full_f = attn.attn_shard_fwd(X, np.hstack([Wq, Wk, Wv]), Wo, nh, d, b, s, causal)
    full_b = attn.attn_shard_bwd(X, np.hstack([Wq, Wk, Wv]), Wo, dZ, nh, d, b, s, causal)
    h = nh * d
    Os, Zs, dXs = [], 0, 0
    for r in range(t):
        Wqkv_r, Wo_r, n = _rank_weights(Wq, Wk, Wv, Wo, t, r, nh, d)
        f = attn.attn_shard_fwd(X, Wqkv_r, Wo_r, n, d, b, s, causal)
        g = attn.attn_shard_bwd(X, Wqkv_r, Wo_r, dZ, n, d, b, s, causal)
        Os.append(f["O"]); Zs = Zs + f["Z"]; dXs = dXs + g["dX"]
        c = slice(r * n * d, (r + 1) * n * d)
        want_dWqkv = np.hstack([full_b["dWqkv"][:, blk * h:(blk + 1) * h][:, c] for blk in range(3)])
        assert rel_fro(g["dWqkv"], want_dWqkv) < 1e-13
        assert rel_fro(g["dWo"], full_b["dWo"][c, :]) < 1e-13
    assert rel_fro(np.hstack(Os), full_f["O"]) < 1e-13
    assert rel_fro(Zs, full_f["Z"]) < 1e-13
    assert rel_fro(dXs, full_b["dX"]) < 1e-13


def test_attn_split_inside_heads_is_wrong(rng):
    """Negative control: splitting each head's d dimensions across ranks (columns
    that do not follow head boundaries) does not give the unsharded output."""
    b, s, nh, d = 2, 6, 4, 4
    X, Wq, Wk, Wv, Wo, _ = _problem(rng, b, s, nh, d)
    full = attn.attn_shard_fwd(X, np.hstack([Wq, Wk, Wv]), Wo, nh, d, b, s, True)["Z"]
    Zs = 0
    for r in range(2):  # rank r takes half of every head's dimensions
        cols = np.concatenate([np.arange(j * d + r * d // 2, j * d + (r + 1) * d // 2) for j in range(nh)])
        Wqkv_r = np.hstack([Wq[:, cols], Wk[:, cols], Wv[:, cols]])
        Zs = Zs + attn.attn_shard_fwd(X, Wqkv_r, Wo[cols, :], nh, d // 2, b, s, True)["Z"]
    assert rel_fro(Zs, full) > 1e-2


@pytest.mark.parametrize("causal", [True, False])
def test_attn_bwd_finite_differences(rng, causal):
    """Central differences of sum(dZ * Z) with respect to X, Wqkv and W_O."""
    b, s, n, d = 2, 3, 2, 2
    X, Wq, Wk, Wv, Wo, dZ = _problem(rng, b, s, n, d, scale_w=0.8)
    Wqkv = np.hstack([Wq, Wk, Wv])

    def obj(Xv, Wv_, Wov):
        return float((attn.attn_shard_fwd(Xv, Wv_, Wov, n, d, b, s, causal)["Z"] * dZ).sum())

    g = attn.attn_shard_bwd(X, Wqkv, Wo, dZ, n, d, b, s, causal)
    eps = 1e-6
    for name, arr, call in (("dX", X, lambda a: obj(a, Wqkv, Wo)), ("dWqkv", Wqkv, lambda a: obj(X, a, Wo)),
                            ("dWo", Wo, lambda a: obj(X, Wqkv, a))):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(*arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            fd[idx] = (call(p) - call(m)) / (2 * eps)
        assert rel_fro(g[name], fd) < 1e-7, name


@pytest.mark.parametrize("causal", [True, False])
def test_attn_uniform_attention_closed_form(rng, causal):
    """W_Q = 0 makes every score 0: each query averages the values it may see (the
    running mean under the causal mask, the sequence mean without it), and the
    row statistic is ln(number of visible keys)."""
    b, s, nh, d = 2, 5, 2, 3
    X, _, Wk, Wv, Wo, _ = _problem(rng, b, s, nh, d)
    fw = attn.attn_shard_fwd(X, np.hstack([np.zeros_like(Wk), Wk, Wv]), Wo, nh, d, b, s, causal)
    V = X @ Wv
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        Vs = V[rows]
        want = np.cumsum(Vs, axis=0) / np.arange(1, s + 1)[:, None] if causal else np.tile(Vs.mean(axis=0), (s, 1))
        np.testing.assert_allclose(fw["O"][rows], want, rtol=1e-13, atol=1e-15)
        cnt = np.arange(1, s + 1) if causal else np.full(s, s)
        np.testing.assert_allclose(fw["lse"][:, rows], np.tile(np.log(cnt), (nh, 1)), rtol=1e-14, atol=1e-15)
    if causal:  # the first position sees only itself
        np.testing.assert_allclose(fw["O"][0::s], V[0::s], rtol=1e-14)


def test_attn_scalar_brute_force(rng):
    """Pure-Python loops (math.exp, math.fsum) for the forward of a causal shard."""
    b, s, n, d = 2, 3, 2, 2
    h = n * d
    X, Wq, Wk, Wv, Wo, _ = _problem(rng, b, s, n, d)

    def mm(A, B):
        return [[math.fsum(A[i][k] * B[k][j] for k in range(len(B))) for j in range(len(B[0]))] for i in range(len(A))]

    Xl = X.tolist()
    Q, K, V = mm(Xl, Wq.tolist()), mm(Xl, Wk.tolist()), mm(Xl, Wv.tolist())
    O = [[0.0] * h for _ in range(b * s)]
    for bi in range(b):
        for j in range(n):
            for q in range(s):
                tq = bi * s + q
                sc = [math.fsum(Q[tq][j * d + e] * K[bi * s + k][j * d + e] for e in range(d)) / math.sqrt(d)
                      for k in range(q + 1)]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = math.fsum(w)
                for e in range(d):
                    O[tq][j * d + e] = math.fsum(w[k] * V[bi * s + k][j * d + e] for k in range(q + 1)) / tot
    Z = mm(O, Wo.tolist())
    fw = attn.attn_shard_fwd(X, np.hstack([Wq, Wk, Wv]), Wo, n, d, b, s, True)
    np.testing.assert_allclose(fw["O"], O, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fw["Z"], Z, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------- mutation checks
def test_pins_catch_missing_scale(rng, monkeypatch):
    orig = attn.attention_core

    def bad(Q, K, V, n, d, b, s, causal):
        return orig(np.asarray(Q) * math.sqrt(d), K, V, n, d, b, s, causal)  # undoes 1/sqrt(d)

    monkeypatch.setattr(attn, "attention_core", bad)
    with pytest.raises(AssertionError):
        test_attn_matches_torch_sdpa_and_autograd(rng, True)


def test_pins_catch_reversed_mask(rng, monkeypatch):
    def bad(s, causal):
        if not causal:
            return np.zeros((s, s))
        q = np.arange(s)[:, None]
        k = np.arange(s)[None, :]
        return np.where(k < q, -np.inf, 0.0)  # a query sees itself and later keys

    monkeypatch.setattr(attn, "_mask", bad)
    with pytest.raises(AssertionError):
        test_attn_uniform_attention_closed_form(rng, True)


def test_pins_catch_softmax_over_queries(rng, monkeypatch):
    def bad(S):
        St = S.T
        mx = np.where(np.isfinite(St), St, -np.inf).max(axis=1, keepdims=True)
        e = np.exp(St - mx)
        tot = e.sum(axis=1, keepdims=True)
        return (e / tot).T, (mx + np.log(tot))[:, 0]  # normalised over the wrong axis

    monkeypatch.setattr(attn, "_softmax_rows", bad)
    with pytest.raises(AssertionError):
        test_attn_scalar_brute_force(rng)


def test_pins_catch_swapped_k_and_v(rng, monkeypatch):
    def bad(QKV, n, d):
        nd = n * d
        return QKV[:, :nd], QKV[:, 2 * nd:], QKV[:, nd:2 * nd]

    monkeypatch.setattr(attn, "_split_qkv", bad)
    with pytest.raises(AssertionError):
        test_attn_matches_torch_sdpa_and_autograd(rng, False)
