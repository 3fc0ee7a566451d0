"""The library's calls inside a HIP graph: forward, backward and split-KV decode are
captured once and replayed several times, with eager work between the replays, and
every replay must equal the eager results bit for bit. No entry point records a
memset or allocates, so a captured call is a plain sequence of kernel launches."""
import pytest

import synthetic
from gpu_util import device, to_dev

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import (attention, attention_backward, bwd_workspace_bytes,  # noqa: E402
                                          decode, decode_workspace_bytes)


def test_forward_backward_decode_replay_in_a_graph():
    import torch
    dev = device()
    B, N, Hq, Hkv, d = 2, 300, 8, 2, 128
    bits = [synthetic.normal_bits(4000, t, (B, N, h, d), "bf16") for t, h in ((0, Hq), (1, Hkv), (2, Hkv), (3, Hq))]
    q, k, v, do = (to_dev(x, "bf16") for x in bits)
    qd = to_dev(synthetic.normal_bits(4001, 0, (B, 1, Hq, d), "bf16"), "bf16")
    # eager reference
    o_e, lse_e = attention(q, k, v, causal=True)
    g_e = attention_backward(q, k, v, o_e, lse_e, do, causal=True)
    od_e, ld_e = decode(qd, k, v, num_splits=8)
    # static buffers for the graph
    o, lse = torch.empty_like(o_e), torch.empty_like(lse_e)
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    od, ld = torch.empty_like(od_e), torch.empty_like(ld_e)
    wsb = torch.empty(bwd_workspace_bytes(B, N, Hq), dtype=torch.uint8, device=dev)
    wsd = torch.empty(decode_workspace_bytes(B, 1, Hq, d, 8), dtype=torch.uint8, device=dev)

    def step():
        attention(q, k, v, causal=True, out=o, lse=lse)
        attention_backward(q, k, v, o, lse, do, causal=True, workspace=wsb, dq=dq, dk=dk, dv=dv)
        decode(qd, k, v, num_splits=8, workspace=wsd, out=od, lse=ld)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv, od, ld, wsb, wsd):
            t.view(torch.uint8).fill_(0xFF)   # poison outputs and workspaces between replays
        junk = torch.randn(1 << 20, device=dev).sum()   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for a, b in ((o, o_e), (dq, g_e[0]), (dk, g_e[1]), (dv, g_e[2]), (od, od_e)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}"
        for a, b in ((lse, lse_e), (ld, ld_e)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"replay {rep}"
