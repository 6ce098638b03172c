"""Steady-state decode window (kv_window_plan / kv_window_upload / kv_window_step) on the
GPU: every step appends one token to each branch and decodes all branches.

- each step's outputs against the fp64 oracle, which appends the same tokens one round
  at a time and decodes over the materialised contexts (bf16 outputs max-abs 2e-2 and
  mean-abs 2e-3, LSE max-abs 2e-3, as for fork_attn_decode);
- the window's steps captured once in a HIP graph and replayed on a second, identical
  pool give the eager outputs bit for bit;
- the page table after the window equals the oracle's (block tables, positions), and a
  second window continues from it.
The branches share a partial tail page (the prefix is not page-aligned), so the first
step writes into copies, and the window crosses page boundaries.  The timed steady-state
workload runs at full size too: 16 branches over a 32,768-token prefix + 2,048 private
tokens each, a 16-step window captured in one HIP graph and replayed once; its first
and last steps against the oracle.
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import build_device_pool, check_close, check_decode_both, out_to_f64, to_torch

pytestmark = pytest.mark.gpu


def _inputs(sc, n, n_steps, seed):
    rng = np.random.default_rng(seed)
    d, hkv, hq = sc.head_dim, sc.n_kv_heads, sc.n_q_heads
    k = [W.to_bf16_bits(rng.standard_normal((n, hkv, d)) / np.sqrt(d)) for _ in range(n_steps)]
    v = [W.to_bf16_bits(rng.standard_normal((n, hkv, d))) for _ in range(n_steps)]
    q = [W.to_bf16_bits(rng.standard_normal((n, hq, d))) for _ in range(n_steps)]
    return k, v, q


def _run(fa, pool, seqs, sc, n_steps, kt, vt, qt, outs, lses, graph):
    import torch
    ws = pool.window(seqs, sc.n_q_heads, n_steps)
    torch.cuda.synchronize()
    if not graph:
        for s in range(n_steps):
            pool.window_step(s, kt[s], vt[s], qt[s], sc.sm_scale, outs[s], lses[s])
        torch.cuda.synchronize()
        return ws
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for s in range(n_steps):
            pool.window_step(s, kt[s], vt[s], qt[s], sc.sm_scale, outs[s], lses[s])
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    return ws, g


def test_window_steps_oracle_graph_and_page_table():
    import torch
    import fork_attention_decode_amd as fa
    from oracle import attention as att, pagetable as pt
    sc = W.fork_scenario(prefix=517, branches=4, private=[0, 3, 16, 30], hq=8, hkv=2, d=128, seed=73)
    sc.n_pages += 48
    seqs, n_steps = [1, 2, 3, 4], 20
    n = len(seqs)
    print(f"[case] window: {n} branches, {n_steps} steps, shared partial tail", flush=True)
    kb, vb, qb = _inputs(sc, n, n_steps, 74)
    kt = [to_torch(x, "bf16") for x in kb]
    vt = [to_torch(x, "bf16") for x in vb]
    qt = [to_torch(x, "bf16") for x in qb]
    res = {}
    keep = []
    for mode in ("eager", "graph"):
        pool, _ = build_device_pool(sc)
        outs = [torch.empty((n, sc.n_q_heads, sc.head_dim), dtype=torch.bfloat16, device="cuda")
                for _ in range(n_steps)]
        lses = [torch.empty((n, sc.n_q_heads), dtype=torch.float32, device="cuda") for _ in range(n_steps)]
        keep.append(_run(fa, pool, seqs, sc, n_steps, kt, vt, qt, outs, lses, mode == "graph"))
        res[mode] = (pool, [o.clone() for o in outs], [l.clone() for l in lses])
    for s in range(n_steps):
        assert torch.equal(res["eager"][1][s], res["graph"][1][s]) and torch.equal(res["eager"][2][s],
                                                                                   res["graph"][2][s]), s
    print("[ok] graph replay equals the eager steps", flush=True)

    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    f = W.bf16_bits_to_f64
    for s in range(n_steps):
        for i, b in enumerate(seqs):
            table.append(b, 1, k=f(kb[s][i:i + 1]), v=f(vb[s][i:i + 1]))
        ref = att.decode(table, seqs, f(qb[s]), sc.sm_scale, with_magnitudes=True)
        o = out_to_f64(res["eager"][1][s], "bf16")
        check_decode_both(o, res["eager"][2][s].double().cpu().numpy(), ref, 128, "bf16", f"window step {s}")
    print(f"[ok] {n_steps} steps against the oracle", flush=True)
    pool = res["eager"][0]
    for b in seqs:
        assert list(pool.block_table(b)) == table.block_table(b), b
        assert np.array_equal(pool.positions(b), table.positions(b)), b
    print("[ok] page table after the window", flush=True)
    # a second window continues from the first
    kb2, vb2, qb2 = _inputs(sc, n, 3, 75)
    outs = [torch.empty((n, sc.n_q_heads, sc.head_dim), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    lses = [torch.empty((n, sc.n_q_heads), dtype=torch.float32, device="cuda") for _ in range(3)]
    _run(fa, pool, seqs, sc, 3, [to_torch(x, "bf16") for x in kb2], [to_torch(x, "bf16") for x in vb2],
         [to_torch(x, "bf16") for x in qb2], outs, lses, False)
    for s in range(3):
        for i, b in enumerate(seqs):
            table.append(b, 1, k=f(kb2[s][i:i + 1]), v=f(vb2[s][i:i + 1]))
        ref = att.decode(table, seqs, f(qb2[s]), sc.sm_scale, with_magnitudes=True)
        check_decode_both(out_to_f64(outs[s], "bf16"), lses[s].double().cpu().numpy(), ref, 128, "bf16", f"second window step {s}")
    print("[ok] a second window continues from the first", flush=True)


def test_long_window_items_past_the_cut():
    # page-aligned prefix, a branch with no private tokens: its window pages form a
    # private segment split into several work items, and at early steps the last items
    # lie wholly past the cut (every slot range empty)
    import torch
    import fork_attention_decode_amd as fa
    from oracle import attention as att, pagetable as pt
    sc = W.fork_scenario(prefix=512, branches=2, private=[0, 5], hq=8, hkv=2, d=128, seed=76)
    sc.n_pages += 40
    seqs, n_steps = [1, 2], 200
    n = len(seqs)
    print(f"[case] window: {n} branches, {n_steps} steps from a page-aligned fork", flush=True)
    kb, vb, qb = _inputs(sc, n, n_steps, 77)
    pool, _ = build_device_pool(sc)
    outs = [torch.empty((n, sc.n_q_heads, sc.head_dim), dtype=torch.bfloat16, device="cuda") for _ in range(n_steps)]
    lses = [torch.empty((n, sc.n_q_heads), dtype=torch.float32, device="cuda") for _ in range(n_steps)]
    _run(fa, pool, seqs, sc, n_steps, [to_torch(x, "bf16") for x in kb], [to_torch(x, "bf16") for x in vb],
         [to_torch(x, "bf16") for x in qb], outs, lses, False)
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    f = W.bf16_bits_to_f64
    check = {0, 1, 15, 16, 17, 100, 199}
    for s in range(n_steps):
        for i, b in enumerate(seqs):
            table.append(b, 1, k=f(kb[s][i:i + 1]), v=f(vb[s][i:i + 1]))
        if s in check:
            ref = att.decode(table, seqs, f(qb[s]), sc.sm_scale, with_magnitudes=True)
            check_decode_both(out_to_f64(outs[s], "bf16"), lses[s].double().cpu().numpy(), ref, 128, "bf16", f"long window step {s}")
    print(f"[ok] steps {sorted(check)} against the oracle", flush=True)


def test_one_step_window_and_an_empty_sequence():
    # a window of one step over a fork and a new, empty root (its first token opens its
    # first page)
    import torch
    import fork_attention_decode_amd as fa
    from oracle import attention as att, pagetable as pt
    sc = W.fork_scenario(prefix=48, branches=1, private=[5], hq=8, hkv=2, d=128, seed=78)
    sc.n_pages += 8
    sc.ops.append(("create",))  # sequence 2, no tokens
    seqs = [2, 1]
    n = len(seqs)
    print("[case] one-step window over an empty root and a fork", flush=True)
    kb, vb, qb = _inputs(sc, n, 1, 79)
    pool, _ = build_device_pool(sc)
    outs = [torch.empty((n, sc.n_q_heads, sc.head_dim), dtype=torch.bfloat16, device="cuda")]
    lses = [torch.empty((n, sc.n_q_heads), dtype=torch.float32, device="cuda")]
    _run(fa, pool, seqs, sc, 1, [to_torch(kb[0], "bf16")], [to_torch(vb[0], "bf16")], [to_torch(qb[0], "bf16")],
         outs, lses, False)
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    f = W.bf16_bits_to_f64
    for i, b in enumerate(seqs):
        table.append(b, 1, k=f(kb[0][i:i + 1]), v=f(vb[0][i:i + 1]))
    ref = att.decode(table, seqs, f(qb[0]), sc.sm_scale, with_magnitudes=True)
    check_decode_both(out_to_f64(outs[0], "bf16"), lses[0].double().cpu().numpy(), ref, 128, "bf16", "one-step window")
    print("[ok] one-step window", flush=True)


def test_window_full_size():
    import torch
    import fork_attention_decode_amd as fa
    from oracle import attention as att, pagetable as pt
    sc = W.shared_prefix_fork()
    sc.n_pages += 64
    seqs, n_steps = list(sc.queries), 16
    n = len(seqs)
    print(f"[case] window, full size: {n} branches, {n_steps} steps in one graph", flush=True)
    kb, vb, qb = _inputs(sc, n, n_steps, 80)
    pool, _ = build_device_pool(sc)
    outs = [torch.empty((n, sc.n_q_heads, sc.head_dim), dtype=torch.bfloat16, device="cuda") for _ in range(n_steps)]
    lses = [torch.empty((n, sc.n_q_heads), dtype=torch.float32, device="cuda") for _ in range(n_steps)]
    keep = _run(fa, pool, seqs, sc, n_steps, [to_torch(x, "bf16") for x in kb], [to_torch(x, "bf16") for x in vb],
                [to_torch(x, "bf16") for x in qb], outs, lses, True)
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    f = W.bf16_bits_to_f64
    for s in range(n_steps):
        for i, b in enumerate(seqs):
            table.append(b, 1, k=f(kb[s][i:i + 1]), v=f(vb[s][i:i + 1]))
        if s in (0, n_steps - 1):
            ref = att.decode(table, seqs, f(qb[s]), sc.sm_scale, with_magnitudes=True)
            check_decode_both(out_to_f64(outs[s], "bf16"), lses[s].double().cpu().numpy(), ref, 128, "bf16", f"full-size window step {s}")
            print(f"[ok] full-size window step {s}", flush=True)
    for b in seqs:
        assert list(pool.block_table(b)) == table.block_table(b), b
    del keep
