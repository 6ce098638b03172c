"""Pins for the packed DAG prefill oracle (CPU only).

* one segment, no edges reduces to plain causal attention: the mask is the lower
  triangle and the output matches torch's fp64 causal scaled_dot_product_attention;
* a hand-written mask for a small DAG;
* exact block-pair and token-pair counts for the packed workload, from closed-form
  arithmetic over the workload's structure (and, at reduced size, from the mask);
* brute force with Python loops on a tiny DAG.
"""
import math

import numpy as np
import torch

import workloads as W
from oracle import prefill as pf


def test_single_segment_is_causal():
    rng = np.random.default_rng(0)
    T, hq, hkv, d = 40, 4, 2, 8
    seg = np.array([[0, T, -1]]); edges = np.zeros((0, 4), int)
    assert np.array_equal(pf.visible_mask(seg, edges, T), np.tril(np.ones((T, T), bool)))
    q, k, v = rng.standard_normal((T, hq, d)), rng.standard_normal((T, hkv, d)), rng.standard_normal((T, hkv, d))
    o, lse = pf.attend_rows(q, k, v, seg, edges, list(range(T)), 0.3)
    rep = lambda x: torch.from_numpy(np.repeat(x.transpose(1, 0, 2), hq // hkv, 0))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q.transpose(1, 0, 2))[None], rep(k),
                                                           rep(v), is_causal=True, scale=0.3)
    assert np.allclose(o, ref[0].numpy().transpose(1, 0, 2), atol=1e-12, rtol=0)


def test_hand_written_dag_mask():
    # prefix [0,2); branch A = segment 1 [2,5); branch B = segment 2 [5,8); edge A[0:2) -> B
    seg = np.array([[0, 2, -1], [2, 3, 0], [5, 3, 0]])
    edges = np.array([[1, 0, 2, 2]])
    exp = np.array([
        # 0  1  2  3  4  5  6  7
        [1, 0, 0, 0, 0, 0, 0, 0],
        [1, 1, 0, 0, 0, 0, 0, 0],
        [1, 1, 1, 0, 0, 0, 0, 0],
        [1, 1, 1, 1, 0, 0, 0, 0],
        [1, 1, 1, 1, 1, 0, 0, 0],
        [1, 1, 1, 1, 0, 1, 0, 0],
        [1, 1, 1, 1, 0, 1, 1, 0],
        [1, 1, 1, 1, 0, 1, 1, 1],
    ], bool)
    assert np.array_equal(pf.visible_mask(seg, edges, 8), exp)
    assert pf.visible_count(seg, edges, 8) == exp.sum()


def closed_form_counts(prefix, branches, blen, n_edges, elen, blk):
    nbp, nbb, neb = prefix // blk, blen // blk, elen // blk
    blocks = nbp * (nbp + 1) // 2 + branches * nbb * nbp + branches * nbb * (nbb + 1) // 2 + n_edges * nbb * neb
    tokens = (prefix * (prefix + 1) // 2 + branches * blen * prefix + branches * blen * (blen + 1) // 2
              + n_edges * blen * elen)
    return blocks, tokens


def test_full_workload_counts():
    p = W.dag_prefill(with_data=False)
    blocks, tokens = closed_form_counts(16384, 8, 8192, 12, 2048, 64)
    assert (blocks, tokens) == (410240, 1677762560)
    assert len(p.edges) == 12 and len({(int(s), int(t)) for s, _, _, t in p.edges}) == 12
    assert all(int(s) < int(t) for s, _, _, t in p.edges)       # source earlier in sync order
    assert pf.visible_count(p.segments, p.edges, p.T) == tokens
    assert 4 * 128 * 32 * tokens == 27488461783040               # FLOPs = 4 d Hq pairs


def test_reduced_workload_block_counts_from_mask():
    p = W.prefill_inputs(prefix=256, branches=4, branch_len=128, n_edges=3, edge_len=64, block=32,
                         with_data=False)
    blocks, tokens = closed_form_counts(256, 4, 128, 3, 64, 32)
    need = pf.block_pairs(p.segments, p.edges, p.T, 32)
    assert need.sum() == blocks
    assert pf.visible_mask(p.segments, p.edges, p.T).sum() == tokens == pf.visible_count(p.segments, p.edges, p.T)


def test_brute_force_tiny_dag():
    rng = np.random.default_rng(7)
    p = W.prefill_inputs(prefix=5, branches=3, branch_len=[4, 3, 6], n_edges=2, edge_len=2, block=1,
                         hq=2, hkv=1, d=4, seed=1)
    T = p.T
    q = W.storage_to_f64(p.q, "bf16"); k = W.storage_to_f64(p.k, "bf16"); v = W.storage_to_f64(p.v, "bf16")
    o, lse = pf.attend_rows(q, k, v, p.segments, p.edges, list(range(T)), 1.0)
    starts = [int(s) for s, _, _ in p.segments]
    for i in range(T):
        si = max(j for j in range(len(starts)) if starts[j] <= i)
        vis = []
        for j in range(T):
            sj = max(x for x in range(len(starts)) if starts[x] <= j)
            ok = (sj == si and j <= i) or (si > 0 and sj == 0)
            for s, off, ln, t in p.edges:
                if t == si and starts[s] + off <= j < starts[s] + off + ln:
                    ok = True
            if ok:
                vis.append(j)
        for h in range(2):
            sc = [sum(q[i, h, c] * k[j, 0, c] for c in range(4)) for j in vis]
            m = max(sc); e = [math.exp(x - m) for x in sc]; z = sum(e)
            ob = [sum(e[a] * v[j, 0, c] for a, j in enumerate(vis)) / z for c in range(4)]
            assert np.allclose(o[i, h], ob, atol=1e-13) and abs(lse[i, h] - (m + math.log(z))) < 1e-12
