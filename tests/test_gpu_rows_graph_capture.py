"""The whole step captured in a HIP graph (through torch.cuda.graphs) and replayed.

The library allocates nothing and clears nothing with memset, so its calls can
be captured.  The graph is replayed several times with eager work and
synchronisations in between, and every replay must reproduce the eager
outputs bit for bit.
"""
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


def test_step_graph_replays_match_eager(ms):
    T, h, f, v = 600, 392, 776, 1000
    print(f"case graph T={T} h={h} f={f} v={v}", flush=True)
    d = inputs.make_inputs(T, h, f, v, bias=True)
    X, A, B, E, dZ, b1 = (_dev(d[k]) for k in ("X", "A", "B", "E", "dZ", "b1"))
    tg = torch.from_numpy(d["targets"]).cuda()
    bf = torch.bfloat16
    H, Y = torch.empty((T, f), dtype=bf, device="cuda"), torch.empty((T, f), dtype=bf, device="cuda")
    Z, dX = torch.empty((T, h), device="cuda"), torch.empty((T, h), device="cuda")
    dA, dB = torch.empty((h, f), dtype=bf, device="cuda"), torch.empty((f, h), dtype=bf, device="cuda")
    db1 = torch.empty((f,), dtype=bf, device="cuda")
    m, s, z = (torch.empty((1, T), device="cuda") for _ in range(3))
    loss, mean = torch.empty((T,), device="cuda"), torch.empty((1,), device="cuda")
    mlp_ws = torch.empty(ms.mlp_shard_workspace_bytes(T, h, f), dtype=torch.uint8, device="cuda")
    ce_ws = torch.empty(ms.vocab_ce_workspace_bytes(T, h, v), dtype=torch.uint8, device="cuda")
    outs = (H, Y, Z, dX, dA, dB, db1, m, s, z, loss, mean)

    def step():
        ms.mlp_shard_fwd(X, A, B, b1, out=(H, Y, Z))
        ms.mlp_shard_bwd(X, A, B, H, Y, dZ, want_db1=True, workspace=mlp_ws, out=(dX, dA, dB, db1))
        ms.vocab_ce_shard_fwd(X, E, tg, 0, workspace=ce_ws, out=(m[0], s[0], z[0]))
        ms.ce_combine(m, s, z, out=(loss, mean))

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream, as torch recommends
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(5):
        for o in outs:
            o.fill_(float("nan")) if o.dtype != torch.bfloat16 else o.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rep, i)
