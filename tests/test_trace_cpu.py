"""The fingerprint tracer's host logic and the fingerprint entry point's validation (CPU).

The tracer is exercised on a stand-in module whose entry points return CPU
tensors, with the oracle's fingerprint as the hash, so its recording, ordering,
restore and comparison logic is checked without a GPU."""
import numpy as np
import pytest
import torch

from oracle import fingerprint as fp

FAKE = 0x7F0000000000


@pytest.fixture(scope="module")
def ms():
    from megatron_tensor_transformer_mlp_amd import mshard
    return mshard


def _cpu_fp(t, chunk):
    f = fp.fingerprint(t.numpy().tobytes(), chunk)
    words = [f["hash"]] + f["chunks"]
    return torch.tensor([w - (1 << 64) if w >= 1 << 63 else w for w in words], dtype=torch.int64)


class _Stub:
    def mlp_shard_fwd(self, x):
        return x + 1, x * 2, None

    def ce_combine(self, x):
        return x.sum(dim=0), x.mean().reshape(1)


def _trace(stub, x, chunks=True):
    from megatron_tensor_transformer_mlp_amd.trace import FingerprintTracer
    with FingerprintTracer(chunk_bytes=64, chunks=chunks, names=("mlp_shard_fwd", "ce_combine"), module=stub,
                           fingerprint_fn=_cpu_fp) as tr:
        stub.mlp_shard_fwd(x)
        stub.ce_combine(x)
        stub.mlp_shard_fwd(x * 3)
    return tr.records


def test_tracer_records_calls_in_order(ms):
    stub = _Stub()
    x = torch.arange(40, dtype=torch.float32).reshape(4, 10)
    recs = _trace(stub, x)
    assert [r["name"] for r in recs] == ["mlp_shard_fwd", "ce_combine", "mlp_shard_fwd"]
    assert [r["call"] for r in recs] == [0, 1, 2]
    o = recs[0]["outputs"]
    assert o[2] is None
    assert o[0]["shape"] == (4, 10) and o[0]["dtype"] == "float32" and o[0]["numel"] == 40
    want = fp.fingerprint((x + 1).numpy().tobytes(), 64)
    assert o[0]["hash"] == f"{want['hash']:016x}"
    assert o[0]["chunks"] == [f"{c:016x}" for c in want["chunks"]] and len(o[0]["chunks"]) == 3
    # entry points are restored on exit
    assert not hasattr(stub.mlp_shard_fwd, "__wrapped__")


def test_tracer_restores_on_exception(ms):
    from megatron_tensor_transformer_mlp_amd.trace import FingerprintTracer
    stub = _Stub()
    with pytest.raises(RuntimeError):
        with FingerprintTracer(names=("mlp_shard_fwd",), module=stub, fingerprint_fn=_cpu_fp):
            raise RuntimeError("boom")
    assert not hasattr(stub.mlp_shard_fwd, "__wrapped__")


def test_first_divergence(ms):
    from megatron_tensor_transformer_mlp_amd.trace import first_divergence
    x = torch.arange(40, dtype=torch.float32).reshape(4, 10)
    a = _trace(_Stub(), x)
    assert first_divergence(a, _trace(_Stub(), x)) is None
    y = x.clone()
    y[3, 9] += 1.0                     # last element: the last 64-byte chunk of the first output
    d = first_divergence(a, _trace(_Stub(), y))
    assert d == {"call": 0, "name": "mlp_shard_fwd", "output": 0, "chunk": 2}
    assert first_divergence(a, a[:2]) == {"call": 2, "name": None, "output": None, "chunk": None}
    b = _trace(_Stub(), x, chunks=False)
    b[1]["outputs"][1]["hash"] = "0" * 16
    assert first_divergence(_trace(_Stub(), x, chunks=False), b) == {"call": 1, "name": "ce_combine", "output": 1,
                                                                     "chunk": None}


def test_fingerprint_words_and_validation(ms):
    assert ms.fingerprint_words(0, 64) == 2
    assert ms.fingerprint_words(1, 64) == 2
    assert ms.fingerprint_words(64, 64) == 2
    assert ms.fingerprint_words(65, 64) == 3
    assert ms.fingerprint_words(100, 7) == 0 and ms.fingerprint_words(100, 0) == 0
    assert ms.fingerprint_words(1 << 40, 8) == 0          # 2^37 chunks
    L = ms.LIB
    assert L.ms_fingerprint(FAKE, 1024, 7, FAKE + (1 << 30), None) == ms.MS_ERR_SHAPE
    assert L.ms_fingerprint(None, 1024, 64, FAKE + (1 << 30), None) == ms.MS_ERR_NULL
    assert L.ms_fingerprint(FAKE, 1024, 64, None, None) == ms.MS_ERR_NULL
    assert L.ms_fingerprint(FAKE + 4, 1024, 64, FAKE + (1 << 30), None) == ms.MS_ERR_ALIGN
    assert L.ms_fingerprint(FAKE, 1024, 64, FAKE + (1 << 30) + 4, None) == ms.MS_ERR_ALIGN
    assert L.ms_fingerprint(FAKE, 1024, 64, FAKE + 1000, None) == ms.MS_ERR_ALIAS
    assert "overlaps" in L.ms_last_error().decode()
