"""fp64 CPU oracle for one tensor-parallel rank's self-attention shard.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code with the HIP library.

Sources (web pages; citations name the page and the section):
  [EXPL]  Megatron-LM explainer, azimuth.plus/paper/megatron-lm, "attention":
          heads are independent computations; the Q, K and V projection
          matrices are split along their columns so each rank computes a
          subset of the heads (16 heads on 4 GPUs: 4 each); the output
          projection O is split by rows, like B of the MLP, so the heads'
          partial outputs enter it with no synchronisation and one all-reduce
          follows it.
  [NOTES] Megatron-LM paper notes, notes.yuuk.io, "self-attention block split":
          K/Q/V GEMMs column-parallel per head, output projection row-parallel
          and reduced across GPUs; with the MLP, four all-reduces per layer.

Readings where the pages are silent (each one is also listed in the design notes):
  * The per-head computation is scaled dot-product attention,
    softmax(Q K^T / sqrt(d) + mask) V over the tokens of one sequence
    (Vaswani et al., "Attention Is All You Need"); the pages only name heads.
  * The mask is causal (a query sees keys at its own and earlier positions)
    for the GPT-like and BLOOM-like layers and absent for the BERT-like one.
  * No biases and no dropout inside the shard (as for the MLP shard).
  * Layout per rank: T = b*s token rows, sequence-major (row = sequence*s +
    position); Wqkv_i [h x 3nd] = [W_Q,i | W_K,i | W_V,i], each block holding
    this rank's n heads of d columns, head-major; W_O,i [nd x h] holds the
    matching rows of W_O.  The shard's output Z_i = O_i W_O,i is this rank's
    fp32 partial (g sums it); its input gradient dX_i is the partial f sums.
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np

from .ref import _f64


def _mask(s: int, causal: bool) -> np.ndarray:
    """Additive mask [s, s]: -inf where key position k > query position q (causal), else 0."""
    if not causal:
        return np.zeros((s, s))
    q = np.arange(s)[:, None]
    k = np.arange(s)[None, :]
    return np.where(k > q, -np.inf, 0.0)


def _softmax_rows(S: np.ndarray):
    mx = S.max(axis=1, keepdims=True)
    e = np.exp(S - mx)
    tot = e.sum(axis=1, keepdims=True)
    return e / tot, (mx + np.log(tot))[:, 0]


def _split_qkv(QKV: np.ndarray, n: int, d: int):
    nd = n * d
    return QKV[:, :nd], QKV[:, nd:2 * nd], QKV[:, 2 * nd:]


def attention_core(Q, K, V, n: int, d: int, b: int, s: int, causal: bool) -> Dict[str, np.ndarray]:
    """Per sequence and head: O = softmax(Q K^T / sqrt(d) + mask) V.

    Q, K, V: [b*s, n*d] (head j in columns j*d .. j*d+d-1).  Returns O [b*s, n*d]
    and lse [n, b*s], the log of each softmax row's normaliser (the statistic a
    recomputing backward needs)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    scale = 1.0 / math.sqrt(d)
    M = _mask(s, causal)
    O = np.zeros_like(Q)
    lse = np.zeros((n, b * s))
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for j in range(n):
            cols = slice(j * d, (j + 1) * d)
            P, l = _softmax_rows(Q[rows, cols] @ K[rows, cols].T * scale + M)
            O[rows, cols] = P @ V[rows, cols]
            lse[j, rows] = l
    return {"O": O, "lse": lse}


def attn_shard_fwd(X, Wqkv_i, Wo_i, n: int, d: int, b: int, s: int, causal: bool) -> Dict[str, np.ndarray]:
    """[EXPL attention] / [NOTES self-attention block split]: this rank's heads.

        [Q | K | V] = X Wqkv_i,   O_i = per-head attention,   Z_i = O_i W_O,i  (partial of g)."""
    X, Wqkv_i, Wo_i = _f64(X), _f64(Wqkv_i), _f64(Wo_i)
    QKV = X @ Wqkv_i
    Q, K, V = _split_qkv(QKV, n, d)
    core = attention_core(Q, K, V, n, d, b, s, causal)
    return {"QKV": QKV, "O": core["O"], "lse": core["lse"], "Z": core["O"] @ Wo_i}


def attn_shard_bwd(X, Wqkv_i, Wo_i, dZ, n: int, d: int, b: int, s: int, causal: bool) -> Dict[str, np.ndarray]:
    """Chain rule through the shard, with dZ arriving unchanged through g's backward.

        dO = dZ W_O,i^T,  dW_O,i = O^T dZ;  per sequence and head, with P the softmax:
        dV = P^T dO_j,  dP = dO_j V_j^T,  dS = P * (dP - rowsum(dP * P)),
        dQ_j = dS K_j / sqrt(d),  dK_j = dS^T Q_j / sqrt(d);
        dWqkv_i = X^T [dQ | dK | dV],  dX_i = [dQ | dK | dV] Wqkv_i^T  (partial of f)."""
    X, Wqkv_i, Wo_i, dZ = _f64(X), _f64(Wqkv_i), _f64(Wo_i), _f64(dZ)
    QKV = X @ Wqkv_i
    Q, K, V = _split_qkv(QKV, n, d)
    O = attention_core(Q, K, V, n, d, b, s, causal)["O"]
    dO = dZ @ Wo_i.T
    scale = 1.0 / math.sqrt(d)
    M = _mask(s, causal)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for j in range(n):
            cols = slice(j * d, (j + 1) * d)
            q, k, v, do = Q[rows, cols], K[rows, cols], V[rows, cols], dO[rows, cols]
            P, _ = _softmax_rows(q @ k.T * scale + M)
            dV[rows, cols] = P.T @ do
            dP = do @ v.T
            dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
            dQ[rows, cols] = dS @ k * scale
            dK[rows, cols] = dS.T @ q * scale
    dQKV = np.hstack([dQ, dK, dV])
    return {"dO": dO, "dQKV": dQKV, "dWo": O.T @ dZ, "dWqkv": X.T @ dQKV, "dX": dQKV @ Wqkv_i.T}
