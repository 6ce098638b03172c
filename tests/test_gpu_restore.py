"""Restoring spans with one prefill (kv_append of segments with their own positions, then
kv_causal_attend over the appended tokens) against the fp64 oracle
(oracle/attention.causal_last): token j sees the own tokens through itself, then the
mounts.  Bars as for decode: bf16 outputs max-abs 2e-2 and mean-abs 2e-3, LSE max-abs
2e-3.  Cases: two segments with positions far apart appended to a fork whose tail page
is shared (copy-on-write), a thread with mounts, a single token, a whole fresh
sequence (plain causal attention, several work-item groups), and the timed restore
workload at full size (sampled tokens, every head).
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import build_device_pool, check_close, out_to_f64, to_torch

pytestmark = pytest.mark.gpu


def _restore(sc, seq, seg_lens, seg_pos, seed, label, rows=None):
    import torch
    from oracle import attention as att, pagetable as pt
    print(f"[case] {label}: segments {seg_lens} at positions {seg_pos}", flush=True)
    rng = np.random.default_rng(seed)
    d, hkv, hq = sc.head_dim, sc.n_kv_heads, sc.n_q_heads
    pool, _ = build_device_pool(sc)
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    f = W.bf16_bits_to_f64
    for n, p0 in zip(seg_lens, seg_pos):
        kb = W.to_bf16_bits(rng.standard_normal((n, hkv, d)) / np.sqrt(d))
        vb = W.to_bf16_bits(rng.standard_normal((n, hkv, d)))
        pos = np.arange(p0, p0 + n, dtype=np.int64)
        pool.append(seq, k=to_torch(kb, "bf16"), v=to_torch(vb, "bf16"), positions=pos)
        table.append(seq, n, k=f(kb), v=f(vb), pos=pos)
    n_all = int(sum(seg_lens))
    qb = W.to_bf16_bits(rng.standard_normal((n_all, hq, d)))
    out, lse = pool.causal_attend(seq, to_torch(qb, "bf16"), sc.sm_scale)
    torch.cuda.synchronize()
    o, l = out_to_f64(out, "bf16"), lse.double().cpu().numpy()
    if rows is not None:
        o, l = o[rows], l[rows]
    ro, rl = att.causal_last(table, seq, f(qb), sc.sm_scale, rows=rows)
    mx, mn = check_close(o, ro, 2e-2, 2e-3, label)
    check_close(l, rl, 2e-3, 2e-3, label + " lse")
    assert np.array_equal(pool.positions(seq), table.positions(seq))
    print(f"[ok] {label}: {len(o)} of {n_all} tokens, max-abs {mx:.3g} mean-abs {mn:.3g}", flush=True)


def test_restore_two_segments_into_a_fork():
    sc = W.fork_scenario(prefix=517, branches=3, private=[40, 0, 9], hq=8, hkv=2, d=128, seed=92)
    sc.n_pages += 16
    _restore(sc, 2, [30, 21], [2000, 4000], 93, "two segments into a fork")


def test_restore_into_a_thread_with_mounts():
    sc = W.dag_scenario(root=300, threads=3, private=90, mounts_per_thread=2, mount_len=33, hq=8, hkv=2, d=128,
                        seed=94)
    sc.n_pages += 16
    _restore(sc, 2, [17, 1, 40], [700, 900, 1200], 95, "segments into a thread with mounts")


def test_single_token_and_fresh_sequence():
    sc = W.fork_scenario(prefix=64, branches=1, private=[3], hq=8, hkv=2, d=128, seed=96)
    sc.n_pages += 40
    _restore(sc, 1, [1], [500], 97, "one token")
    # a new root (id 2) filled by one segment of 300 tokens: plain causal attention
    sc.ops.append(("create",))
    _restore(sc, 2, [300], [0], 98, "fresh sequence, 300 tokens")


def test_restore_full_size():
    # the timed restore workload: 4 segments of 128 tokens, positions 100,000 apart, into
    # one branch of the shared-prefix pool (32,768-token prefix + 2,048 private tokens),
    # then one causal attention of the 512 restored tokens over the 35,328-token context
    # (16,384 query rows); the first and last tokens of every segment and a few between
    sc = W.shared_prefix_fork()
    sc.n_pages += 64
    rows = [0, 1, 63, 127, 128, 200, 255, 256, 320, 383, 384, 450, 510, 511]
    _restore(sc, sc.queries[0], [128] * 4, [100000, 200000, 300000, 400000], 99, "restore, full size", rows=rows)
