"""GPU parity of the library's buffer fingerprints against the plain-Python oracle,
and the fingerprint tracer on real library calls.

Fingerprints are integers, so the bar is exact equality.
"""
import numpy as np
import pytest
import torch

from megatron_tensor_transformer_mlp_amd import inputs
from oracle import fingerprint as fp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ms():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from megatron_tensor_transformer_mlp_amd import mshard
    return mshard


def _words(t):
    return [int(x) & ((1 << 64) - 1) for x in t.cpu().tolist()]


@pytest.mark.parametrize("n,chunk", [(0, 64), (1, 8), (7, 64), (8, 8), (31, 64), (32, 64), (33, 64), (1000, 32),
                                     (4096, 4096), (65536 + 5, 4096), (3 << 20, 1 << 16), (1 << 20, 1 << 20)])
def test_fingerprint_matches_oracle(ms, n, chunk):
    print(f"case fingerprint n={n} chunk={chunk}", flush=True)
    data = np.random.Generator(np.random.PCG64(n)).integers(0, 256, size=n, dtype=np.uint8)
    t = torch.from_numpy(data).cuda()
    got = _words(ms.fingerprint(t, chunk))
    want = fp.fingerprint(data.tobytes(), chunk)
    assert got[1:] == want["chunks"]
    assert got[0] == want["hash"]


def test_fingerprint_of_tensor_views_and_dtypes(ms):
    """The bytes of a bf16 and an int64 tensor, as stored."""
    d = inputs.make_inputs(64, 64, 256, 512)
    X = torch.from_numpy(d["X"].view(np.int16)).view(torch.bfloat16).cuda()
    assert _words(ms.fingerprint(X, 1024))[0] == fp.fingerprint(d["X"].tobytes(), 1024)["hash"]
    tg = torch.from_numpy(d["targets"]).cuda()
    assert _words(ms.fingerprint(tg, 64))[0] == fp.fingerprint(d["targets"].tobytes(), 64)["hash"]


def test_tracer_on_library_calls(ms):
    """Two identical runs trace identically; a one-element change in dZ first shows
    in the backward call, in the outputs that depend on it."""
    from megatron_tensor_transformer_mlp_amd.trace import FingerprintTracer, first_divergence
    d = inputs.make_inputs(600, 392, 776, 1000, bias=True)

    def dev(u):
        return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).cuda()

    def run(dZ_bits):
        X, A, B, E, b1 = dev(d["X"]), dev(d["A"]), dev(d["B"]), dev(d["E"]), dev(d["b1"])
        tg = torch.from_numpy(d["targets"]).cuda()
        with FingerprintTracer(chunks=True) as tr:
            H, Y, Z = ms.mlp_shard_fwd(X, A, B, b1)
            ms.mlp_shard_bwd(X, A, B, H, Y, dev(dZ_bits), want_db1=True)
            m, s, z = ms.vocab_ce_shard_fwd(X, E, tg, 0)
            ms.ce_combine(m[None], s[None], z[None])
        return tr.records

    a = run(d["dZ"])
    assert first_divergence(a, run(d["dZ"])) is None
    dz = d["dZ"].copy()
    dz[599, 391] ^= 0x0001                       # last element of dZ
    div = first_divergence(a, run(dz))
    assert div["call"] == 1 and div["name"] == "mlp_shard_bwd"
