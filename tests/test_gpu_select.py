"""GPU parity of key scoring (kv_score), keep selection (kv_select_keep) and the drop that
follows (kv_drop_keep), against the fp64 oracle (oracle/select.py).

Bars: scores within 2e-4 relative (+1e-9 absolute) of the fp64 scores, from the fp32
arithmetic on the same bf16 inputs: each probability is exp2(s c2 - lse2); the exponent
s c2 is a 128-term fp32 dot product of exact bf16 products (worst case 128 u times
sum |q_i k_i| c2 ~ 10, i.e. ~8e-5 absolute in log2 units), and the normaliser is a sum
of at most a few thousand terms per lane merged in a shallow tree (~1e-5 relative), so
each probability, and their mean, is within ~1e-4 relative; measured errors are below
1e-6.  Keep masks are bit-exact against the oracle's selection applied to the GPU's own
fp32 scores (the decision is taken in the same precision on both sides).  After the
drop, the page table is bit-exact and the decode is within the decode bars.
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import build_device_pool, check_close, check_decode_both, oracle_decode, out_to_f64, to_torch

pytestmark = pytest.mark.gpu

REL, ABS = 2e-4, 1e-9


def _q_rep(n_rep, hq, d, seed):
    # representative queries: seeded N(0,1) draws, one rounding to bf16 (fed to both sides)
    return W.to_bf16_bits(np.random.default_rng(seed).standard_normal((n_rep, hq, d)))


def _oracle_table(sc):
    from oracle import pagetable as pt
    return pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))


def _scores(sc, seq, n_rep, seed, label):
    import torch
    from oracle import select as sel
    print(f"[case] {label}: seq {seq}, {n_rep} representative queries", flush=True)
    pool, _ = build_device_pool(sc)
    qb = _q_rep(n_rep, sc.n_q_heads, sc.head_dim, seed)
    got = pool.score(seq, to_torch(qb, "bf16"), sc.sm_scale)
    torch.cuda.synchronize()
    got = got.double().cpu().numpy()
    table, _ = _oracle_table(sc)
    ref = sel.key_scores(table, seq, W.bf16_bits_to_f64(qb), sc.sm_scale)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    bad = err > REL * ref + ABS
    assert not bad.any(), f"{label}: {int(bad.sum())} scores off, worst rel {float((err / (ref + 1e-30)).max()):.3g}"
    print(f"[ok] {label}: n={len(ref)} max rel {float((err / (ref + 1e-30)).max()):.3g} sum {got.sum():.6f}",
          flush=True)
    return pool, got, ref


@pytest.mark.parametrize("n_rep,private", [(1, 37), (8, 300), (16, 130), (32, 1000)])
def test_scores_fork(n_rep, private):
    # a fork over a shared prefix: the fork's own context is prefix + private tokens; 4, 32, 64
    # and 128 rows per KV head (1, 2, 4 and 8 row tiles)
    sc = W.fork_scenario(prefix=517, branches=2, private=[private, 5], hq=8, hkv=2, d=128, seed=41)
    _, got, ref = _scores(sc, 1, n_rep, 42, f"scores n_rep={n_rep} private={private}")
    assert abs(got.sum() - 1.0) < 1e-2  # no mounts: every softmax sums to 1


def test_scores_d64_and_many_rows():
    # head dim 64, G = 8 and 32 queries: 256 rows per KV head, the most one launch takes
    sc = W.fork_scenario(prefix=200, branches=1, private=[90], hq=16, hkv=2, d=64, seed=43)
    _scores(sc, 1, 32, 44, "scores d=64, 256 rows per KV head")


def test_scores_with_mounts():
    sc = W.dag_scenario(root=300, threads=3, private=90, mounts_per_thread=2, mount_len=33, hq=8, hkv=2, d=128,
                        seed=45)
    _, got, _ = _scores(sc, 2, 8, 46, "scores of a thread with mounts")
    assert 0.0 < got.sum() < 1.0  # mounted keys take part of the mass and are not scored


@pytest.mark.parametrize("n", [1, 1000, 131072])
def test_select_keep_exact(n):
    import torch
    import fork_attention_decode_amd as fa
    from oracle import select as sel
    rng = np.random.default_rng(47 + n)
    # quantised values: many exact ties around every threshold
    sc = (rng.integers(0, max(2, n // 50), size=n) / 7.0).astype(np.float32)
    sc[rng.random(n) < 0.01] = 0.0
    t = torch.from_numpy(sc).cuda()
    for budget in sorted({0, 1, n // 3, n // 2, n - 1, n, n + 5}):
        print(f"[case] select n={n} budget={budget}", flush=True)
        keep = fa.select_keep(t, budget)
        torch.cuda.synchronize()
        got = keep.cpu().numpy().astype(bool)
        want = sel.select_keep(sc.astype(np.float64), budget)
        assert np.array_equal(got, want), f"n={n} budget={budget}: {int((got != want).sum())} entries differ"


@pytest.mark.parametrize("kind", ["all_equal", "signed_zeros"])
def test_select_keep_ties_across_slices(kind):
    # the threshold's ties span many workgroup slices and must still go in index order
    import torch
    import fork_attention_decode_amd as fa
    from oracle import select as sel
    rng = np.random.default_rng(51)
    if kind == "all_equal":
        n = 300_001
        sc = np.full(n, 0.25, np.float32)
    else:
        n = 70_001
        sc = rng.choice(np.array([-1.5, -0.0, 0.0, 0.5, 2.0], np.float32), size=n)
    t = torch.from_numpy(sc).cuda()
    for budget in (1, n // 2, n - 1):
        print(f"[case] select {kind} n={n} budget={budget}", flush=True)
        got = fa.select_keep(t, budget).cpu().numpy().astype(bool)
        want = sel.select_keep(sc.astype(np.float64), budget)
        assert np.array_equal(got, want), f"{kind} budget={budget}: {int((got != want).sum())} entries differ"


@pytest.mark.parametrize("repos", [True, False])
def test_select_drop_then_decode(repos):
    import torch
    from oracle import select as sel
    sc = W.fork_scenario(prefix=700, branches=2, private=[900, 40], hq=8, hkv=2, d=128, seed=48)
    sc.n_pages += 60
    pool, _ = build_device_pool(sc)
    qb = _q_rep(16, sc.n_q_heads, sc.head_dim, 49)
    n_own = pool.info(1)[0]
    budget = int(0.6 * n_own)
    print(f"[case] score + keep {budget} of {n_own} + drop (repos={repos}) + decode", flush=True)
    keep = pool.select_and_drop(1, to_torch(qb, "bf16"), sc.sm_scale, budget, repos=repos)
    torch.cuda.synchronize()
    assert int(keep.sum()) == budget
    # several keep sets are correct where fp32 scores tie to within their rounding: the
    # GPU's set must be one of them by the oracle's fp64 scores (no dropped key scores
    # above a kept one by more than the score bar), and the oracle then drops its spans
    ref = sel.key_scores(_oracle_table(sc)[0], 1, W.bf16_bits_to_f64(qb), sc.sm_scale)
    kb = keep.astype(bool)
    assert ref[~kb].max() <= ref[kb].min() + 2 * (REL * ref[kb].min() + ABS), "keep set not a top-k of the scores"
    sc.ops = sc.ops + [("drop", 1, sel.drop_spans(kb), repos)]
    table, _ = _oracle_table(sc)
    assert list(pool.block_table(1)) == table.block_table(1)
    assert np.array_equal(pool.positions(1), table.positions(1))
    for p in range(sc.n_pages):
        assert pool.refcount(p) == table.rc[p], f"refcount of page {p}"
    out, lse = pool.decode(sc.queries, to_torch(sc.q, "bf16"), sc.sm_scale)
    torch.cuda.synchronize()
    check_decode_both(out_to_f64(out, "bf16"), lse.double().cpu().numpy(), oracle_decode(sc, with_magnitudes=True),
                      sc.head_dim, "bf16", "decode after select + drop", rerotated_keys=repos)
    print("[ok] select + drop + decode", flush=True)


def test_scores_full_size():
    """One 131,072-token sequence (32 / 8 heads, d = 128), 32 representative queries: every
    score against the oracle, and the keep mask at 60 % against the oracle's selection
    on the GPU scores."""
    import torch
    import fork_attention_decode_amd as fa
    from oracle import select as sel
    sc = W.fork_scenario(prefix=131072 - 16, branches=1, private=[16], hq=32, hkv=8, d=128, seed=3)
    pool, got, ref = _scores(sc, 1, 32, 50, "scores, 131,072 tokens, 32 queries")
    budget = int(0.6 * len(got))
    keep = fa.select_keep(torch.from_numpy(got.astype(np.float32)).cuda(), budget)
    torch.cuda.synchronize()
    want = sel.select_keep(got.astype(np.float32).astype(np.float64), budget)
    assert np.array_equal(keep.cpu().numpy().astype(bool), want)
