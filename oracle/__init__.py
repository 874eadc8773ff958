"""fp64 CPU oracle (test infrastructure only; never called by the library's product path)."""
from .ref import (bf16_to_f64, ce_combine, ce_row_stats, full_vocab_ce, gelu, gelu_grad,  # noqa: F401
                  mlp_shard_bwd, mlp_shard_fwd, mlp_shard_sampled, vocab_ce_shard, vocab_ce_shard_bwd)
from . import attn  # noqa: F401,E402  (self-attention shard)
from . import fingerprint  # noqa: F401,E402  (buffer fingerprints)
