"""Restoring spans with one prefill (kv_append of segments with their own positions, then
kv_causal_attend over the appended tokens) against the fp64 oracle
(oracle/attention.causal_last): token j sees the own tokens through itself, then the
mounts.  Bars as for decode: bf16 outputs max-abs 2e-2 and mean-abs 2e-3, LSE max-abs
2e-3.  Cases: two segments with positions far apart appended to a fork whose tail page
is shared (copy-on-write), a thread with mounts (misaligned: K relaid; page-aligned: K
gathered from the pool), a single token, a whole fresh
sequence (plain causal attention, several work-item groups), fp32 and d = 64 pools (the
decode-row path), and the timed restore workload at full size (sampled tokens, every
head).  Bars: also the error model's (tests/harness.py: decode_bars), with the tiled
prefill's row sum over the rounded P for bf16 / d = 128 pools.
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import build_device_pool, check_decode_both, out_to_f64, to_torch

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
    dt = sc.dtype
    store = (lambda x: W.to_bf16_bits(x)) if dt == "bf16" else (lambda x: x.astype(np.float32))
    f = (lambda a: W.storage_to_f64(a, dt))
    for n, p0 in zip(seg_lens, seg_pos):
        kb = store(rng.standard_normal((n, hkv, d)) / np.sqrt(d))
        vb = store(rng.standard_normal((n, hkv, d)))
        pos = np.arange(p0, p0 + n, dtype=np.int64)
        pool.append(seq, k=to_torch(kb, dt), v=to_torch(vb, dt), positions=pos)
        table.append(seq, n, k=f(kb), v=f(vb), pos=pos)
    n_all = int(sum(seg_lens))
    qb = store(rng.standard_normal((n_all, hq, d)))
    out, lse = pool.causal_attend(seq, to_torch(qb, dt), sc.sm_scale)
    torch.cuda.synchronize()
    o, l = out_to_f64(out, dt), lse.double().cpu().numpy()
    if rows is not None:
        o, l = o[rows], l[rows]
    ref = att.causal_last(table, seq, f(qb), sc.sm_scale, rows=rows, with_magnitudes=True)
    # bf16 pools with d = 128 restore by the tiled prefill (row sums over the rounded P,
    # accumulator chains of up to 4,096 steps); others by rows of the split-K decode
    tiled = dt == "bf16" and d == 128
    mx, mn, wo, wl = check_decode_both(o, l, ref, d, dt, label, gamma=2.0 ** -12 if tiled else None,
                                       rounded_p_sum=tiled)
    assert np.array_equal(pool.positions(seq), table.positions(seq))
    print(f"[ok] {label}: {len(o)} of {n_all} tokens, max-abs {mx:.3g} mean-abs {mn:.3g}; error / model bar: "
          f"O {wo:.3f}, LSE {wl:.3f}", flush=True)


def test_restore_two_segments_into_a_fork():
    sc = W.fork_scenario(prefix=517, branches=3, private=[40, 0, 9], hq=8, hkv=2, d=128, seed=92)
    sc.n_pages += 16
    _restore(sc, 2, [30, 21], [2000, 4000], 93, "two segments into a fork")


def test_restore_into_a_thread_with_mounts():
    sc = W.dag_scenario(root=300, threads=3, private=90, mounts_per_thread=2, mount_len=33, hq=8, hkv=2, d=128,
                        seed=94)
    sc.n_pages += 16
    _restore(sc, 2, [17, 1, 40], [700, 900, 1200], 95, "segments into a thread with mounts")


def test_restore_into_a_thread_with_page_aligned_mounts():
    # mounts that start on page boundaries and span whole pages, own context a multiple of
    # 16 after the restore: every visible 16-key group is one page, so K is gathered
    # straight from the pool (the misaligned mounts above take the relayout)
    sc = W.dag_scenario(root=304, threads=3, private=96, mounts_per_thread=2, mount_len=32, hq=8, hkv=2, d=128,
                        seed=88)
    sc.n_pages += 16
    _restore(sc, 2, [17, 1, 46], [700, 900, 1200], 89, "segments into a thread with page-aligned mounts")


def test_single_token_and_fresh_sequence():
    sc = W.fork_scenario(prefix=64, branches=1, private=[3], hq=8, hkv=2, d=128, seed=96)
    sc.n_pages += 40
    _restore(sc, 1, [1], [500], 97, "one token")
    # a new root (id 2) filled by one segment of 300 tokens: plain causal attention
    sc.ops.append(("create",))
    _restore(sc, 2, [300], [0], 98, "fresh sequence, 300 tokens")


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_restore_random_shapes(seed):
    # seeded random shapes: forks (even seeds) or threads with mounts (odd seeds, page-aligned
    # or not), head counts, and 1 .. 4 segments of random lengths (restored spans from one
    # token to several 64-token row groups, own contexts ending anywhere in a page)
    rng = np.random.default_rng(3000 + seed)
    hq, hkv = [(8, 2), (4, 1), (16, 4), (8, 8)][seed]
    if seed % 2 == 0:
        sc = W.fork_scenario(prefix=int(rng.integers(1, 1500)), branches=2,
                             private=[int(x) for x in rng.integers(0, 200, size=2)], hq=hq, hkv=hkv, d=128,
                             seed=60 + seed)
        seq = 1
    else:
        aligned = seed == 3
        private = 16 * int(rng.integers(3, 12)) if aligned else int(rng.integers(40, 200))
        sc = W.dag_scenario(root=16 * int(rng.integers(1, 60)) if aligned else int(rng.integers(1, 900)), threads=3,
                            private=private, mounts_per_thread=2,
                            mount_len=16 * int(rng.integers(1, private // 16 + 1)) if aligned
                            else int(rng.integers(1, private + 1)), hq=hq, hkv=hkv, d=128, seed=60 + seed)
        seq = 2
    n_seg = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 120, size=n_seg)]
    pos = [5000 * (i + 1) + int(rng.integers(0, 1000)) for i in range(n_seg)]
    sc.n_pages += 64
    _restore(sc, seq, lens, pos, 70 + seed, f"random restore seed={seed} Hq={hq} Hkv={hkv}")


@pytest.mark.parametrize("dtype,d", [("f32", 128), ("bf16", 64)])
def test_restore_by_decode_rows(dtype, d):
    # pools the tiled prefill does not take (fp32, d = 64) restore as rows of the split-K
    # decode; a fork with mounts-free context, two segments
    sc = W.fork_scenario(prefix=333, branches=2, private=[20, 50], hq=8, hkv=2, d=d, dtype=dtype, rope_theta=1e4,
                         seed=91)
    sc.n_pages += 16
    _restore(sc, 2, [70, 9], [3000, 5000], 90, f"restore {dtype} d={d} by decode rows")


def test_restore_full_size():
    # the timed restore workload: 4 segments of 128 tokens, positions 100,000 apart, into
    # one branch of the shared-prefix pool (32,768-token prefix + 2,048 private tokens),
    # then one causal attention of the 512 restored tokens over the 35,328-token context
    # (16,384 query rows); the first and last tokens of every segment and a few between
    sc = W.shared_prefix_fork()
    sc.n_pages += 64
    rows = [0, 1, 63, 127, 128, 200, 255, 256, 320, 383, 384, 450, 510, 511]
    _restore(sc, sc.queries[0], [128] * 4, [100000, 200000, 300000, 400000], 99, "restore, full size", rows=rows)
