"""Decode steps replayed from a HIP graph give the eager result.

A serving loop (and bench.py's timed region) captures fork_attn_partials +
fork_attn_merge, whose plans are cached after the first call, in a HIP graph and
replays it.  Each replay here runs with eager decode work and host synchronisation
between replays, and its outputs must equal the eager outputs bit for bit (same
kernels, same inputs, same order).  Every case prints its name first.
"""
import pytest

import workloads as W
from tests.harness import build_device_pool, to_torch

pytestmark = pytest.mark.gpu


def _step(fa, pool, ws, sc, hq, q, out, lse, stream):
    fa.fork_attn_partials(pool.handle, sc.queries, hq, q.data_ptr(), sc.sm_scale, ws.data_ptr(), ws.numel(), stream)
    fa.fork_attn_merge(pool.handle, sc.queries, hq, out.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(), stream)


@pytest.mark.parametrize("name", ["tiny_fork_decode", "shared_prefix_fork_decode"])
def test_graph_replay_equals_eager(name):
    import torch
    import fork_attention_decode_amd as fa
    sc = W.WORKLOADS[name]()
    print(f"[case] graph replay: {name}", flush=True)
    pools = [build_device_pool(sc)[0] for _ in range(2)]
    q = to_torch(sc.q, sc.dtype)
    n, hq, _ = q.shape
    wss = [torch.zeros(fa.fork_attn_workspace_size(p.handle, sc.queries, hq), dtype=torch.uint8, device="cuda")
           for p in pools]
    outs = [torch.empty_like(q) for _ in pools]
    lses = [torch.empty((n, hq), dtype=torch.float32, device="cuda") for _ in pools]
    s0 = torch.cuda.current_stream().cuda_stream
    for i in range(2):  # eager reference (and the plans cached for each pool / workspace)
        _step(fa, pools[i], wss[i], sc, hq, q, outs[i], lses[i], s0)
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        s = torch.cuda.current_stream().cuda_stream
        for i in range(2):
            _step(fa, pools[i], wss[i], sc, hq, q, outs[i], lses[i], s)
    torch.cuda.synchronize()
    for rep in range(3):
        for o, l in zip(outs, lses):
            o.zero_()
            l.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], ref[i][0]) and torch.equal(lses[i], ref[i][1]), f"replay {rep}, pool {i}"
        _step(fa, pools[0], wss[0], sc, hq, q, outs[0], lses[0], s0)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(outs[0], ref[0][0])
        print(f"[ok] replay {rep}", flush=True)
