"""Shared helpers of the GPU parity tests and the bench: replay a ``workloads`` scenario
through the library on the device, and through the oracle on the CPU."""
from __future__ import annotations

import numpy as np

import workloads as W


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def out_to_f64(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return W.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


def build_device_pool(sc: W.Scenario, extra_pages: int = 0, stream_sync: bool = True):
    """Replay the scenario's operations on a device pool.  Returns (pool, kept lists)."""
    import torch
    import fork_attention_decode_amd as fa
    pool = fa.Pool(sc.n_kv_heads, sc.head_dim, sc.n_pages + extra_pages, dtype=sc.dtype,
                   rope_theta=sc.rope_theta)
    kept = []
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "append":
            blk = sc.blocks[op[2]]
            k = to_torch(blk.k, sc.dtype)
            v = to_torch(blk.v, sc.dtype)
            pool.append(op[1], k, v, positions=blk.pos)
            if stream_sync:
                torch.cuda.synchronize()  # keep k / v alive until the copy kernel ran
        elif op[0] == "fork":
            pool.fork(op[1])
        elif op[0] == "mount":
            pool.mount(*op[1:])
        elif op[0] == "drop":
            kept.append(pool.drop(op[1], op[2], repos=op[3]))
        elif op[0] == "release":
            pool.release(op[1])
    torch.cuda.synchronize()
    return pool, kept


def oracle_decode(sc: W.Scenario, rows=None):
    """fp64 oracle outputs (o [n, Hq, d], lse [n, Hq]) for the scenario's queries (or the
    listed query indices)."""
    from oracle import attention as att, pagetable as pt
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    q = W.storage_to_f64(sc.q, sc.dtype)
    idx = list(range(len(sc.queries))) if rows is None else list(rows)
    o, lse = att.decode(table, [sc.queries[i] for i in idx], q[idx], sc.sm_scale)
    return o, lse


def subscenario(sc: W.Scenario, seq_ids):
    """The operations of independent sequences `seq_ids` only (creation order kept), with
    sequence ids renumbered; used to run the oracle one request at a time."""
    remap = {}
    ops = []
    blocks = []
    nxt = 0
    owner = []
    for op in sc.ops:  # ids in creation order
        if op[0] in ("create", "fork"):
            owner.append(op)
    sid = 0
    keep_ops = []
    for op in sc.ops:
        if op[0] == "create":
            if sid in seq_ids:
                remap[sid] = nxt
                nxt += 1
                keep_ops.append(("create",))
            sid += 1
        elif op[0] == "fork":
            raise ValueError("subscenario is for independent sequences")
        elif op[1] in remap:
            if op[0] == "append":
                blocks.append(sc.blocks[op[2]])
                keep_ops.append(("append", remap[op[1]], len(blocks) - 1))
            else:
                keep_ops.append((op[0], remap[op[1]]) + tuple(op[2:]))
    qi = [sc.queries.index(s) for s in seq_ids]
    sub = W.Scenario(name=sc.name + "_sub", n_q_heads=sc.n_q_heads, n_kv_heads=sc.n_kv_heads, head_dim=sc.head_dim,
                     page_size=sc.page_size, dtype=sc.dtype, sm_scale=sc.sm_scale, rope_theta=sc.rope_theta,
                     n_pages=sc.n_pages, ops=keep_ops, blocks=blocks, queries=[remap[s] for s in seq_ids],
                     q=sc.q[qi])
    return sub


def check_close(got: np.ndarray, ref: np.ndarray, max_abs: float, mean_abs: float, what: str = ""):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mn = float(err.max()), float(err.mean())
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3g} (<= {max_abs}), mean-abs {mn:.3g} (<= {mean_abs})"
    return mx, mn
