"""fp64 CPU oracle for one tensor-parallel rank's MLP shard and vocab-parallel CE shard.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library: it reads the same seeded bf16 bit patterns, widens them to
float64 itself and evaluates the plain definitions with numpy/scipy.

Sources (web pages; citations name the page and the section):
  [EXPL]  Megatron-LM explainer, azimuth.plus/paper/megatron-lm
          - "core idea: slicing the feed-forward network": Y = GeLU(XA),
            Z = Dropout(YB); A split by columns so GeLU is applied per shard
            with no synchronisation; B split by rows, one all-reduce after it.
          - "the f and g operators": f = identity forward / all-reduce of the
            gradient backward; g = all-reduce forward / identity backward.
  [NOTES] Megatron-LM paper notes, notes.yuuk.io
          - "MLP block split": same column/row split, two GEMMs.
          - "vocab-embedding parallelism": E_{H x v} split along the vocabulary,
            partial GEMMs [XE_1, XE_2], output GEMM fused with cross-entropy so
            the exchange shrinks from b*s*v to b*s.

Readings where the pages are silent (each one is also listed in the design notes):
  * GeLU: the erf definition x*Phi(x) by default; the tanh approximation of the
    GELU paper (Hendrycks & Gimpel) on request.
  * Backward: the chain rule through Y = GeLU(XA_i + b1_i), Z_i = Y B_i with dZ
    replicated on every rank (g's backward is the identity).
  * CE partials: per token, the shard-local max m, the sum of exp(logit - m)
    over the shard s, and the target logit z if the shard owns the target
    (global id in [vocab_start, vocab_start + v_i)), else 0.
  * Combine: M = max_r m_r, S = sum_r s_r exp(m_r - M), loss = ln S + M - sum_r z_r;
    the reported loss is the mean over tokens.
  * Padded vocabulary columns take part in the softmax like any other column.
  * CE backward (the pages give only the forward fusion): the objective is
    sum_t coef[t] * loss[t] (coef = 1/T for the mean); the derivative of a
    token's loss with respect to its logits is the textbook softmax minus the
    one-hot target, with the softmax taken over the whole vocabulary through
    the combined (M, S) of the token.  dX_i is a partial over this rank's
    vocab columns (the ranks' partials sum); dE_i is this rank's own slice.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np
from scipy import special

_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
_TANH_C = 0.044715


# ----------------------------------------------------------------------------- inputs
def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u32 = np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def _f64(a):
    if a is None:
        return None
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


# ----------------------------------------------------------------------------- GeLU
def gelu(x: np.ndarray, form: str = "erf") -> np.ndarray:
    """GeLU(x) = x * Phi(x) (erf form) or the tanh approximation."""
    if form == "erf":
        return 0.5 * x * (1.0 + special.erf(x / math.sqrt(2.0)))
    if form == "tanh":
        return 0.5 * x * (1.0 + np.tanh(_SQRT_2_OVER_PI * (x + _TANH_C * x ** 3)))
    raise ValueError(form)


def gelu_grad(x: np.ndarray, form: str = "erf") -> np.ndarray:
    """d/dx GeLU(x): Phi(x) + x*phi(x) (erf form) or the tanh form's analytic derivative."""
    if form == "erf":
        cdf = 0.5 * (1.0 + special.erf(x / math.sqrt(2.0)))
        pdf = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
        return cdf + x * pdf
    if form == "tanh":
        u = _SQRT_2_OVER_PI * (x + _TANH_C * x ** 3)
        th = np.tanh(u)
        du = _SQRT_2_OVER_PI * (1.0 + 3.0 * _TANH_C * x * x)
        return 0.5 * (1.0 + th) + 0.5 * x * (1.0 - th * th) * du
    raise ValueError(form)


# ----------------------------------------------------------------------------- MLP shard
def mlp_shard_fwd(X, A_i, B_i, b1_i=None, form: str = "erf") -> Dict[str, np.ndarray]:
    """[EXPL core idea] / [NOTES MLP block split]: H = X A_i (+ b1_i), Y = GeLU(H), Z_i = Y B_i.

    Z_i is this rank's partial of Y B; g would sum the partials over ranks.
    Dropout acts after that sum and is not part of the shard.
    """
    X, A_i, B_i, b1_i = _f64(X), _f64(A_i), _f64(B_i), _f64(b1_i)
    H = X @ A_i
    if b1_i is not None:
        H = H + b1_i[None, :]
    Y = gelu(H, form)
    Z = Y @ B_i
    return {"H": H, "Y": Y, "Z": Z}


def mlp_shard_bwd(X, A_i, B_i, dZ, b1_i=None, form: str = "erf") -> Dict[str, np.ndarray]:
    """Chain rule through the shard ([EXPL f and g operators]: dZ arrives unchanged
    through g's backward; dX_i is the partial that f's backward all-reduces).

        dY = dZ B_i^T,  dH = dY * GeLU'(H),  dB_i = Y^T dZ,  dA_i = X^T dH,
        db1_i = sum over tokens of dH,  dX_i = dH A_i^T.
    """
    X, A_i, B_i, dZ, b1_i = _f64(X), _f64(A_i), _f64(B_i), _f64(dZ), _f64(b1_i)
    H = X @ A_i
    if b1_i is not None:
        H = H + b1_i[None, :]
    Y = gelu(H, form)
    dY = dZ @ B_i.T
    dH = dY * gelu_grad(H, form)
    return {"dX": dH @ A_i.T, "dA": X.T @ dH, "dB": Y.T @ dZ,
            "db1": dH.sum(axis=0), "dH": dH}


def mlp_shard_sampled(X, A_i, B_i, dZ, rows: Sequence[int], cols: Sequence[int],
                      b1_i=None, form: str = "erf") -> Dict[str, np.ndarray]:
    """The same definitions evaluated only where they are needed for sampled outputs.

    Per-token outputs on token rows R: H[R,:], Y[R,:], Z[R,:], dH[R,:], dX[R,:]
    (each needs only that token's row).  Per-FFN-column outputs on columns C:
    dA[:,C], dB[C,:], db1[C] (each needs only the columns C of H, Y, dH over
    all tokens).
    """
    X, A_i, B_i, dZ, b1_i = _f64(X), _f64(A_i), _f64(B_i), _f64(dZ), _f64(b1_i)
    R = np.asarray(rows, dtype=np.int64)
    C = np.asarray(cols, dtype=np.int64)
    # token rows
    HR = X[R] @ A_i
    if b1_i is not None:
        HR = HR + b1_i[None, :]
    YR = gelu(HR, form)
    ZR = YR @ B_i
    dHR = (dZ[R] @ B_i.T) * gelu_grad(HR, form)
    dXR = dHR @ A_i.T
    # FFN columns
    HC = X @ A_i[:, C]
    if b1_i is not None:
        HC = HC + b1_i[C][None, :]
    YC = gelu(HC, form)
    dHC = (dZ @ B_i[C, :].T) * gelu_grad(HC, form)
    return {"rows": R, "cols": C, "H_rows": HR, "Y_rows": YR, "Z_rows": ZR, "dH_rows": dHR,
            "dX_rows": dXR, "dA_cols": X.T @ dHC, "dB_cols": YC.T @ dZ, "db1_cols": dHC.sum(axis=0)}


# ----------------------------------------------------------------------------- vocab CE
def vocab_ce_shard(X, E_i, targets, vocab_start: int, rows: Optional[Sequence[int]] = None,
                   block: int = 512) -> Dict[str, np.ndarray]:
    """[NOTES vocab-embedding parallelism]: this rank's logits X E_i reduced per token to
    (m, s, z) so only b*s values per quantity leave the rank.

        m[t] = max_j L[t,j],  s[t] = sum_j exp(L[t,j] - m[t]),
        z[t] = L[t, y_t - vocab_start] if the shard owns y_t else 0.

    ``rows`` restricts the evaluation to those tokens; tokens are processed
    ``block`` at a time only to bound memory (each token is independent).
    """
    X, E_i = _f64(X), _f64(E_i)
    targets = np.asarray(targets, dtype=np.int64)
    R = np.arange(X.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    v_i = E_i.shape[1]
    m = np.empty(len(R)); s = np.empty(len(R)); z = np.empty(len(R))
    for b0 in range(0, len(R), block):
        rb = R[b0:b0 + block]
        L = X[rb] @ E_i
        mb = L.max(axis=1)
        m[b0:b0 + block] = mb
        s[b0:b0 + block] = np.exp(L - mb[:, None]).sum(axis=1)
        loc = targets[rb] - vocab_start
        own = (loc >= 0) & (loc < v_i)
        zb = np.zeros(len(rb))
        zb[own] = L[np.nonzero(own)[0], loc[own]]
        z[b0:b0 + block] = zb
    return {"m": m, "s": s, "z": z}


def ce_combine(m: np.ndarray, s: np.ndarray, z: np.ndarray) -> Dict[str, np.ndarray]:
    """Merge t shards' partials (arrays [t, T], rank order) into per-token loss and the mean.

        M = max_r m_r,  S = sum_r s_r exp(m_r - M),  loss = ln S + M - sum_r z_r.
    """
    m = np.atleast_2d(np.asarray(m, dtype=np.float64))
    s = np.atleast_2d(np.asarray(s, dtype=np.float64))
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    M = m.max(axis=0)
    S = (s * np.exp(m - M[None, :])).sum(axis=0)
    loss = np.log(S) + M - z.sum(axis=0)
    return {"loss": loss, "mean": math.fsum(loss.tolist()) / loss.size}


def full_vocab_ce(X, E, targets, rows: Optional[Sequence[int]] = None, block: int = 512) -> np.ndarray:
    """Unsharded cross-entropy per token: logsumexp_j (X E)[t,j] - (X E)[t, y_t]."""
    X, E = _f64(X), _f64(E)
    targets = np.asarray(targets, dtype=np.int64)
    R = np.arange(X.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty(len(R))
    for b0 in range(0, len(R), block):
        rb = R[b0:b0 + block]
        L = X[rb] @ E
        out[b0:b0 + block] = special.logsumexp(L, axis=1) - L[np.arange(len(rb)), targets[rb]]
    return out


# ----------------------------------------------------------------------------- vocab CE backward
def ce_row_stats(m, s) -> Dict[str, np.ndarray]:
    """Combined softmax statistics of each token from t shards' partials [t, T]:
    M = max_r m_r and S = sum_r s_r exp(m_r - M), so that the sum over the whole
    vocabulary of exp(L[t, j] - M[t]) is S[t] ([NOTES vocab-embedding parallelism]:
    only these b*s-sized values cross ranks)."""
    m = np.atleast_2d(np.asarray(m, dtype=np.float64))
    s = np.atleast_2d(np.asarray(s, dtype=np.float64))
    M = m.max(axis=0)
    return {"M": M, "S": (s * np.exp(m - M[None, :])).sum(axis=0)}


def _ce_grad_block(L, M, S, coef, targets, vocab_start, cols):
    """dL on a block of logits L[rows, cols]: coef * (softmax - one-hot of the target).

    ``cols`` are the block's column indices within the shard; the target of a row
    sits in this block iff its global id equals vocab_start + a column index."""
    P = np.exp(L - M[:, None]) / S[:, None]
    onehot = ((np.asarray(targets, dtype=np.int64)[:, None] - vocab_start) == np.asarray(cols)[None, :])
    return coef[:, None] * (P - onehot)


def vocab_ce_shard_bwd(X, E_i, targets, vocab_start: int, m, s, coef,
                       rows: Optional[Sequence[int]] = None,
                       cols: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Backward of the fused output GEMM + cross-entropy on one vocab shard.

    Inputs: the shard's X [T, h] and E_i [h, v_i], global target ids, the shard's
    first global column ``vocab_start``, the gathered partials m, s [t, T] of
    every rank (rank order), and the per-token weight coef [T] of the objective
    sum_t coef[t] * loss[t].

        P[t, j]    = exp(L[t, j] - M[t]) / S[t]            (L = X E_i, M, S from ce_row_stats)
        dL_i[t, j] = coef[t] * (P[t, j] - [vocab_start + j == y_t])
        dX_i       = dL_i E_i^T    (this rank's partial; summed over ranks)
        dE_i       = X^T dL_i      (this rank's slice of dE)

    Without rows/cols every output is returned in full.  With them: dX on token
    rows R (each needs only that token's logit row) and dE on shard columns C
    (each needs only that column's logits over all tokens).
    """
    X, E_i = _f64(X), _f64(E_i)
    st = ce_row_stats(m, s)
    M, S = st["M"], st["S"]
    coef = np.broadcast_to(np.asarray(coef, dtype=np.float64), M.shape)
    targets = np.asarray(targets, dtype=np.int64)
    v_i = E_i.shape[1]
    if rows is None and cols is None:
        dL = _ce_grad_block(X @ E_i, M, S, coef, targets, vocab_start, np.arange(v_i))
        return {"dL": dL, "dX": dL @ E_i.T, "dE": X.T @ dL}
    R = np.arange(X.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    C = np.arange(v_i) if cols is None else np.asarray(cols, dtype=np.int64)
    dLR = _ce_grad_block(X[R] @ E_i, M[R], S[R], coef[R], targets[R], vocab_start, np.arange(v_i))
    dLC = _ce_grad_block(X @ E_i[:, C], M, S, coef, targets, vocab_start, C)
    return {"rows": R, "cols": C, "dL_rows": dLR, "dX_rows": dLR @ E_i.T, "dE_cols": X.T @ dLC}
