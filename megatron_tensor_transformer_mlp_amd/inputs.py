"""Seeded synthetic inputs for one tensor-parallel rank's MLP and vocab-CE shards.

This module is the only code shared between the HIP path (its tests and bench)
and the fp64 CPU oracle.  It draws random numbers, scales them and rounds them
to bf16 bit patterns; it contains none of the method's arithmetic.

Recipe (the same bytes feed both sides):
  * ``np.random.SeedSequence(seed).spawn(9)`` gives one child per stream, in
    the fixed order X, A, B, E, dZ, targets, b1, Wqkv, Wo (children are
    positional, so the first seven are those of the original seven-stream
    recipe).  Weight streams (A, B, E, b1, Wqkv, Wo)
    spawn one grandchild per tensor-parallel rank, so rank r's shard is drawn
    directly (entries are iid, which has the same law as slicing a full draw).
  * Normals are drawn as float32 from PCG64, multiplied by a float32 sigma and
    rounded to bf16 with round-to-nearest-even on the bit pattern.  Draws are
    produced in row blocks from one generator, which yields exactly the stream
    a single draw would.
  * Targets are int64 global vocabulary ids, uniform over [0, v_global).

Shapes follow the Megatron-LM paper notes (MLP-block split, self-attention
block split and vocab-embedding parallelism sections): X[T x h], A_i[h x f_i],
B_i[f_i x h], E_i[h x v_i], dZ[T x h], Wqkv_i[h x 3nd], Wo_i[nd x h], all
row-major.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

STREAMS = ("X", "A", "B", "E", "dZ", "targets", "b1", "Wqkv", "Wo")
_ELEMS_PER_BLOCK = 1 << 24


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round-to-nearest-even; NaN kept quiet.

    For every non-NaN pattern u <= 0xFF800000, u + 0x7FFF + 1 fits in 32 bits.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u + np.uint32(0x7FFF)
    r += (u >> np.uint32(16)) & np.uint32(1)
    r >>= np.uint32(16)
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class ShardConfig:
    """One rank's shard shapes: T tokens, hidden h, FFN columns f_i, vocab columns v_i."""
    name: str
    T: int
    h: int
    f_i: int
    v_i: int
    t: int                # tensor-parallel degree the shard belongs to
    v_global: int         # full (padded) vocabulary size
    sigma_w: float = 0.02  # std of A, B, E (and b1)
    bias: bool = False

    @property
    def mlp_flop(self) -> int:
        """fwd 2 GEMMs + bwd 4 GEMMs, each 2*T*h*f_i."""
        return 12 * self.T * self.h * self.f_i

    @property
    def ce_flop(self) -> int:
        return 2 * self.T * self.h * self.v_i


# The five workloads: a tiny full layer, a GPT-2 1.5B-like full layer (t=1),
# an 8.3B-GPT-like rank shard (t=8), a 3.9B-BERT-like rank shard (t=4) and a
# 176B-scale (BLOOM-like) rank shard (t=4).  Vocabularies are padded sizes.
CONFIGS: Dict[str, ShardConfig] = {
    "tiny": ShardConfig("tiny", T=64, h=64, f_i=256, v_i=512, t=1, v_global=512),
    "gpt2_1p5b": ShardConfig("gpt2_1p5b", T=8192, h=1600, f_i=6400, v_i=50304, t=1,
                             v_global=50304),
    "gpt_8p3b_t8": ShardConfig("gpt_8p3b_t8", T=8192, h=3072, f_i=1536, v_i=6400, t=8,
                               v_global=51200),
    "bert_3p9b_t4": ShardConfig("bert_3p9b_t4", T=8192, h=2560, f_i=2560, v_i=7648, t=4,
                                v_global=30592),
    "bloom_176b_t4": ShardConfig("bloom_176b_t4", T=2048, h=14336, f_i=14336, v_i=62720, t=4,
                                 v_global=250880, sigma_w=0.006),
}
CONFIG_ORDER = ["tiny", "gpt2_1p5b", "gpt_8p3b_t8", "bert_3p9b_t4", "bloom_176b_t4"]


def _children(seed: int) -> Dict[str, np.random.SeedSequence]:
    return dict(zip(STREAMS, np.random.SeedSequence(seed).spawn(len(STREAMS))))


def _normal_bf16(ss: np.random.SeedSequence, shape, sigma: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    rows, cols = (shape[0], int(np.prod(shape[1:]))) if len(shape) > 1 else (1, shape[0])
    out = np.empty((rows, cols), dtype=np.uint16)
    s = np.float32(sigma)
    step = max(1, _ELEMS_PER_BLOCK // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = round_to_bf16_bits(g.standard_normal((r1 - r0, cols), dtype=np.float32) * s)
    return out.reshape(shape)


def _rank_child(ss: np.random.SeedSequence, t: int, rank: int) -> np.random.SeedSequence:
    return ss.spawn(t)[rank]


def make_inputs(T: int, h: int, f_i: int, v_i: int, *, t: int = 1, rank: int = 0,
                v_global: Optional[int] = None, sigma_w: float = 0.02, bias: bool = False,
                seed: int = 1234, want=("X", "A", "B", "E", "dZ", "targets", "b1")) -> Dict[str, np.ndarray]:
    """Rank ``rank``'s inputs as bf16 bit patterns (uint16) plus int64 targets.

    Returns a dict with any of: X[T,h], A[h,f_i], B[f_i,h], E[h,v_i], dZ[T,h],
    targets[T] (global ids in [0, v_global)), b1[f_i] (only if ``bias``), and
    ``vocab_start`` = rank * v_i.
    """
    if v_global is None:
        v_global = v_i * t
    ch = _children(seed)
    out: Dict[str, np.ndarray] = {}
    if "X" in want:
        out["X"] = _normal_bf16(ch["X"], (T, h), 1.0)
    if "A" in want:
        out["A"] = _normal_bf16(_rank_child(ch["A"], t, rank), (h, f_i), sigma_w)
    if "B" in want:
        out["B"] = _normal_bf16(_rank_child(ch["B"], t, rank), (f_i, h), sigma_w)
    if "E" in want:
        out["E"] = _normal_bf16(_rank_child(ch["E"], t, rank), (h, v_i), sigma_w)
    if "dZ" in want:
        out["dZ"] = _normal_bf16(ch["dZ"], (T, h), 1.0)
    if "targets" in want:
        g = np.random.Generator(np.random.PCG64(ch["targets"]))
        out["targets"] = g.integers(0, v_global, size=T, dtype=np.int64)
    if bias and "b1" in want:
        out["b1"] = _normal_bf16(_rank_child(ch["b1"], t, rank), (f_i,), sigma_w)
    out["vocab_start"] = np.int64(rank * v_i)
    return out


def make_config_inputs(cfg: ShardConfig, *, rank: int = 0, seed: int = 1234,
                       want=("X", "A", "B", "E", "dZ", "targets", "b1")) -> Dict[str, np.ndarray]:
    return make_inputs(cfg.T, cfg.h, cfg.f_i, cfg.v_i, t=cfg.t, rank=rank, v_global=cfg.v_global,
                       sigma_w=cfg.sigma_w, bias=cfg.bias, seed=seed, want=want)


def sample_indices(n: int, count: int, seed: int, edges: List[int]) -> np.ndarray:
    """Sorted unique sample of [0, n): ``count`` seeded picks plus the given edge indices."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, n, count])))
    pick = g.choice(n, size=min(count, n), replace=False)
    extra = np.array([e for e in edges if 0 <= e < n], dtype=np.int64)
    return np.unique(np.concatenate([pick.astype(np.int64), extra]))


@dataclasses.dataclass(frozen=True)
class AttnConfig:
    """One rank's self-attention shard: b sequences of s tokens, hidden h, n_heads
    heads of size d in the whole layer, t ranks (n_heads / t heads each)."""
    name: str
    b: int
    s: int
    h: int
    n_heads: int
    d: int
    t: int
    causal: bool
    sigma_w: float = 0.02

    @property
    def T(self) -> int:
        return self.b * self.s

    @property
    def n(self) -> int:
        """Heads on one rank."""
        return self.n_heads // self.t


# Attention shards of the same five layers.  The 8.3B-GPT-like shard's head size
# of 96 is the one the paper notes give for their GPT scaling models; the other
# head counts are those of the named models' published configurations.
ATTN_CONFIGS: Dict[str, AttnConfig] = {
    "tiny": AttnConfig("tiny", b=2, s=32, h=64, n_heads=4, d=16, t=1, causal=True),
    "gpt2_1p5b": AttnConfig("gpt2_1p5b", b=8, s=1024, h=1600, n_heads=25, d=64, t=1, causal=True),
    "gpt_8p3b_t8": AttnConfig("gpt_8p3b_t8", b=8, s=1024, h=3072, n_heads=32, d=96, t=8, causal=True),
    "bert_3p9b_t4": AttnConfig("bert_3p9b_t4", b=16, s=512, h=2560, n_heads=40, d=64, t=4, causal=False),
    "bloom_176b_t4": AttnConfig("bloom_176b_t4", b=1, s=2048, h=14336, n_heads=112, d=128, t=4, causal=True,
                                sigma_w=0.006),
}


def make_attn_inputs(b: int, s: int, h: int, n: int, d: int, *, t: int = 1, rank: int = 0,
                     sigma_w: float = 0.02, seed: int = 1234,
                     want=("X", "Wqkv", "Wo", "dZ")) -> Dict[str, np.ndarray]:
    """Rank ``rank``'s attention-shard inputs as bf16 bit patterns (uint16).

    X[b*s, h] and dZ[b*s, h] are the same draws as the MLP shard's for the same
    token count and hidden size; Wqkv[h, 3nd] and Wo[nd, h] come from their
    own streams, one grandchild per rank (n = heads on this rank)."""
    ch = _children(seed)
    T = b * s
    out: Dict[str, np.ndarray] = {}
    if "X" in want:
        out["X"] = _normal_bf16(ch["X"], (T, h), 1.0)
    if "Wqkv" in want:
        out["Wqkv"] = _normal_bf16(_rank_child(ch["Wqkv"], t, rank), (h, 3 * n * d), sigma_w)
    if "Wo" in want:
        out["Wo"] = _normal_bf16(_rank_child(ch["Wo"], t, rank), (n * d, h), sigma_w)
    if "dZ" in want:
        out["dZ"] = _normal_bf16(ch["dZ"], (T, h), 1.0)
    return out


def make_attn_config_inputs(cfg: AttnConfig, *, rank: int = 0, seed: int = 1234,
                            want=("X", "Wqkv", "Wo", "dZ")) -> Dict[str, np.ndarray]:
    return make_attn_inputs(cfg.b, cfg.s, cfg.h, cfg.n, cfg.d, t=cfg.t, rank=rank, sigma_w=cfg.sigma_w, seed=seed,
                            want=want)
