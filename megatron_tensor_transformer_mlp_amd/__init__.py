"""MI355X (gfx950) kernels for one tensor-parallel rank's MLP shard and vocab-parallel CE shard.

The compute entry points live in ``megatron_tensor_transformer_mlp_amd.mshard`` (a thin
ctypes binding over libmshard.so); they are re-exported here lazily so that the seeded
input generator (``.inputs``) can be imported without the library.
"""
_BINDING_NAMES = ("mlp_shard_fwd", "mlp_shard_bwd", "vocab_ce_shard_fwd", "ce_combine",
                  "mlp_shard_workspace_bytes", "vocab_ce_workspace_bytes", "ce_combine_workspace_bytes",
                  "MshardError", "version")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import mshard
        return getattr(mshard, name)
    raise AttributeError(name)
