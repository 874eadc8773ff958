"""Fingerprint tracing of the library's entry points, for finding where two runs
first differ (Megatron Core bitwise-determinism news item, news.hamidun.com,
"debugging methodology": ordered fingerprints of tensors, computed on the GPU
with their shape, dtype and element count, chunk-wise where the order of the
data matters; narrow down from the first differing step to the first
differing call).

    with FingerprintTracer() as tr:
        ... calls through megatron_tensor_transformer_mlp_amd.mshard ...
    records = tr.records            # one dict per call, in call order
    first_divergence(records_a, records_b)

While a tracer is active, the binding's entry points (looked up as
``mshard.<name>`` at call time) are wrapped: after each call, every output
tensor is fingerprinted by the library's own kernel on the current stream.
The fingerprints stay on the device until the tracer exits, so tracing adds
no synchronisation to the traced calls.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence

import torch

from . import mshard as _mshard

TRACED = ("mlp_shard_fwd", "mlp_shard_bwd", "vocab_ce_shard_fwd", "vocab_ce_shard_bwd", "ce_combine",
          "attn_shard_fwd", "attn_shard_bwd")


def _outputs(result) -> List[Optional[torch.Tensor]]:
    if isinstance(result, torch.Tensor):
        return [result]
    return list(result)


class FingerprintTracer:
    """Records, per call of a traced entry point: its index, its name and, for each
    output, shape, dtype, element count, the whole-tensor fingerprint and (with
    ``chunks=True``) the per-chunk fingerprints.  ``module`` and ``fingerprint_fn``
    exist so the recording logic can be exercised without a GPU."""

    def __init__(self, chunk_bytes: int = 1 << 16, chunks: bool = False, names: Sequence[str] = TRACED,
                 module=_mshard, fingerprint_fn: Optional[Callable[[torch.Tensor, int], torch.Tensor]] = None):
        self.chunk_bytes = chunk_bytes
        self.chunks = chunks
        self.names = tuple(names)
        self.module = module
        self.fingerprint_fn = fingerprint_fn or _mshard.fingerprint
        self.records: List[Dict] = []
        self._pending: List[Dict] = []
        self._saved: Dict[str, Callable] = {}

    def _wrap(self, name: str, fn: Callable) -> Callable:
        def traced(*args, **kwargs):
            result = fn(*args, **kwargs)
            outs = []
            for t in _outputs(result):
                if t is None:
                    outs.append(None)
                    continue
                outs.append({"shape": tuple(t.shape), "dtype": str(t.dtype).replace("torch.", ""),
                             "numel": t.numel(), "fp": self.fingerprint_fn(t.contiguous(), self.chunk_bytes)})
            self._pending.append({"call": len(self._pending), "name": name, "outputs": outs})
            return result
        traced.__wrapped__ = fn
        return traced

    def __enter__(self) -> "FingerprintTracer":
        for name in self.names:
            fn = getattr(self.module, name)
            self._saved[name] = fn
            setattr(self.module, name, self._wrap(name, fn))
        return self

    def __exit__(self, *exc) -> None:
        for name, fn in self._saved.items():
            setattr(self.module, name, fn)
        self._saved.clear()
        for rec in self._pending:
            for o in rec["outputs"]:
                if o is None:
                    continue
                words = [int(x) & ((1 << 64) - 1) for x in o.pop("fp").cpu().tolist()]
                o["hash"] = f"{words[0]:016x}"
                if self.chunks:
                    o["chunks"] = [f"{w:016x}" for w in words[1:]]
        self.records.extend(self._pending)
        self._pending = []


def first_divergence(a: Sequence[Dict], b: Sequence[Dict]) -> Optional[Dict]:
    """The first call whose record differs between two traces (name, shapes, dtypes,
    sizes or fingerprints), with the index of the first differing output and, when
    both carry chunk fingerprints, of the first differing chunk.  None if the traces
    agree over their common length and have the same length."""
    for i, (ra, rb) in enumerate(zip(a, b)):
        if ra["name"] != rb["name"] or len(ra["outputs"]) != len(rb["outputs"]):
            return {"call": i, "name": (ra["name"], rb["name"]), "output": None, "chunk": None}
        for j, (oa, ob) in enumerate(zip(ra["outputs"], rb["outputs"])):
            if oa == ob:
                continue
            chunk = None
            if oa and ob and "chunks" in oa and "chunks" in ob:
                chunk = next((k for k, (x, y) in enumerate(zip(oa["chunks"], ob["chunks"])) if x != y), None)
            return {"call": i, "name": ra["name"], "output": j, "chunk": chunk}
    if len(a) != len(b):
        return {"call": min(len(a), len(b)), "name": None, "output": None, "chunk": None}
    return None
