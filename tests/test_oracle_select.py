"""Pins for the key-scoring / keep-selection oracle (CPU only).

key_scores: a scalar brute force on tiny inputs; the closed forms "own scores sum to 1
when nothing is mounted" (every softmax sums to 1) and "identical keys score 1/n"; a
mounted context takes probability mass away from own tokens; a planted key aligned with
every query is the top score.  select_keep / drop_spans: ties go to the lower index,
budget edge cases, spans are maximal and complementary to the kept set.
"""
import math

import numpy as np

from oracle import pagetable as pt, select as sel


def _table(hkv, d, lens, rng, mounts=()):
    t = pt.PageTable(64, 16, hkv, d, with_data=True)
    sids = []
    for n in lens:
        s = t.create()
        t.append(s, n, rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d)))
        sids.append(s)
    for dst, src, b, n in mounts:
        t.mount(sids[dst], sids[src], b, n)
    return t, sids


def _brute(k_rows, q_rep, scale, hq, hkv):
    """k_rows: list over context tokens of [hkv][d] lists; q_rep: [n_rep][hq][d] lists."""
    g = hq // hkv
    n = len(k_rows)
    acc = [0.0] * n
    for qr in q_rep:
        for h in range(hq):
            s = [scale * sum(a * b for a, b in zip(k_rows[t][h // g], qr[h])) for t in range(n)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for t in range(n):
                acc[t] += e[t] / z
    return [x / (len(q_rep) * hq) for x in acc]


def test_scores_brute_force():
    rng = np.random.default_rng(3)
    t, (s,) = _table(2, 4, [21], rng)
    q = rng.standard_normal((3, 4, 4))
    got = sel.key_scores(t, s, q, 0.6)
    k, _ = t.materialise(s)
    want = _brute(k.tolist(), q.tolist(), 0.6, 4, 2)
    assert np.allclose(got, want, atol=1e-15, rtol=0)


def test_scores_sum_to_one_without_mounts():
    rng = np.random.default_rng(4)
    for n in (1, 16, 37, 200):
        t, (s,) = _table(2, 8, [n], rng)
        sc = sel.key_scores(t, s, rng.standard_normal((5, 8, 8)), 0.35)
        assert sc.shape == (n,) and abs(sc.sum() - 1.0) < 1e-12 and (sc > 0).all()


def test_identical_keys_score_one_over_n():
    t = pt.PageTable(8, 16, 1, 4, with_data=True)
    s = t.create()
    n = 23
    kk = np.tile(np.array([0.3, -1.0, 2.0, 0.5]), (n, 1, 1))
    t.append(s, n, kk, np.zeros((n, 1, 4)))
    sc = sel.key_scores(t, s, np.random.default_rng(5).standard_normal((4, 2, 4)), 1.0)
    assert np.allclose(sc, 1.0 / n, atol=1e-15, rtol=0)


def test_mounts_take_mass_and_are_not_scored():
    rng = np.random.default_rng(6)
    t, (a, b) = _table(2, 8, [40, 50], rng, mounts=[(1, 0, 10, 20)])
    sc = sel.key_scores(t, b, rng.standard_normal((4, 4, 8)), 0.35)
    assert sc.shape == (50,) and 0.0 < sc.sum() < 1.0


def test_planted_key_is_top_and_kept():
    rng = np.random.default_rng(7)
    t = pt.PageTable(16, 16, 1, 8, with_data=True)
    s = t.create()
    n = 60
    k = rng.standard_normal((n, 1, 8)) * 0.1
    u = rng.standard_normal(8)
    k[31, 0] = 3.0 * u
    t.append(s, n, k, np.zeros((n, 1, 8)))
    q = np.stack([u + 0.05 * rng.standard_normal(8) for _ in range(6)])[:, None, :].repeat(2, axis=1)
    sc = sel.key_scores(t, s, q, 1.0)
    assert int(np.argmax(sc)) == 31
    for budget in (1, 5, 59):
        assert sel.select_keep(sc, budget)[31]


def test_select_ties_budget_and_spans():
    sc = np.array([0.5, 0.2, 0.5, 0.9, 0.2, 0.2, 0.5, 0.1])
    keep = sel.select_keep(sc, 4)  # 0.9 (t3), then the 0.5s at t0, t2, t6: all of them
    assert keep.tolist() == [True, False, True, True, False, False, True, False]
    keep = sel.select_keep(sc, 5)  # one of the three 0.2s: the lowest index, t1
    assert keep.tolist() == [True, True, True, True, False, False, True, False]
    assert not sel.select_keep(sc, 0).any() and sel.select_keep(sc, 99).all()
    assert sel.select_keep(sc, 5).sum() == 5
    rng = np.random.default_rng(8)
    for _ in range(200):
        keep = rng.random(int(rng.integers(0, 40))) < rng.random()
        spans = sel.drop_spans(keep)
        dropped = np.zeros(len(keep), bool)
        for i, (a, n) in enumerate(spans):
            assert n > 0 and not dropped[a:a + n].any()
            dropped[a:a + n] = True
            assert a == 0 or keep[a - 1]  # maximal on the left
            assert a + n == len(keep) or keep[a + n]  # and on the right
        assert (dropped == ~keep).all()
