"""The allocation-free CE entry point (vocab_ce_shard_fwd_noalloc) against
vocab_ce_shard_fwd, called through the C ABI.

Both run the same kernels, so the outputs must be equal bit for bit.  Two calls
in a row share the GPU's static scratch array, the second with a smaller input
(fewer tokens and vocabulary columns) than the first, so the second reads
partials of its own and none left behind by the first.
"""
import ctypes

import numpy as np
import pytest
import torch

from megatron_tensor_transformer_mlp_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ms():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from megatron_tensor_transformer_mlp_amd import mshard
    return mshard


def _dev(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def _call_noalloc(ms, X, E, tg, T, h, v, start):
    got = [torch.full((T,), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    st = ms.LIB.vocab_ce_shard_fwd_noalloc(X.data_ptr(), E.data_ptr(), tg.data_ptr(), T, h, v, start,
                                           *[g.data_ptr() for g in got], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ms.MS_OK, ms.LIB.ms_last_error().decode()
    return got


def test_noalloc_matches_workspace_entry_two_calls(ms):
    ref = {}
    for T, h, v in [(4100, 392, 1000), (300, 136, 520)]:  # the second call is smaller
        print(f"case noalloc T={T} h={h} v={v}", flush=True)
        d = inputs.make_inputs(T, h, 8, v, t=2, rank=1, v_global=2 * v)
        X, E, tg = _dev(d["X"]), _dev(d["E"]), torch.from_numpy(d["targets"]).cuda()
        want = ms.vocab_ce_shard_fwd(X, E, tg, v)
        got = _call_noalloc(ms, X, E, tg, T, h, v, v)
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        ref[(T, h, v)] = [g.clone() for g in got]
    # and the binding's wrapper of the same entry point, once more on the first shape
    T, h, v = 4100, 392, 1000
    d = inputs.make_inputs(T, h, 8, v, t=2, rank=1, v_global=2 * v)
    X, E, tg = _dev(d["X"]), _dev(d["E"]), torch.from_numpy(d["targets"]).cuda()
    out = tuple(torch.empty((T,), dtype=torch.float32, device="cuda") for _ in range(3))
    ms.vocab_ce_shard_fwd_noalloc(X, E, tg, v, out=out)
    torch.cuda.synchronize()
    for a, b in zip(out, ref[(T, h, v)]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_noalloc_refuses_oversized(ms):
    T, h, v = 1 << 20, 8, 8192  # partials of 32 column tiles x 2^20 tokens x 12 bytes > 32 MiB
    st = ms.LIB.vocab_ce_shard_fwd_noalloc(1 << 40, 2 << 40, 3 << 40, T, h, v, 0, 4 << 40, 5 << 40, 6 << 40, None)
    assert st == ms.MS_ERR_WORKSPACE
    assert "scratch" in ms.LIB.ms_last_error().decode()
