"""Pins for the oracle's page table (CPU only).

The oracle's block tables / refcounts are pinned by
  * the one worked integer example the pages print (Agentrix tool-page sharing),
  * hand-derived cases written out from the rules in the oracle header,
  * invariants (references == refcounts, free + used == capacity, fork allocates
    nothing, a shared page is never written, reclaim only at rc 0),
  * an independent page-free model of every sequence's visible context (plain
    Python lists of token vectors) over random operation sequences.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import pagetable as pt, rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_agentrix_page_sharing_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "agentrix_page_sharing.json")))
    page = 4096                                   # implied by the printed figures
    n_src_pages = g["source_bytes"] // page       # 2048
    t = pt.PageTable(n_pages=n_src_pages * 10, page_size=page)
    src = t.create()
    t.append(src, g["source_bytes"])
    rng = np.random.default_rng(0)
    for b in range(g["branches"]):
        free0 = t.n_free
        c = t.fork(src)
        assert t.n_free == free0                      # fork allocates nothing
        pg = int(rng.integers(0, n_src_pages))
        off = int(rng.integers(0, page - g["edit_chars"] + 1))
        t.write(c, pg * page + off, g["edit_chars"])
    t.check_invariants()
    used = t.capacity - t.n_free
    assert used == n_src_pages + g["branches"] == 2056
    shared_mib = used * page / 2**20
    naive_mib = (1 + g["branches"]) * g["source_bytes"] / 2**20
    assert shared_mib == g["unique_payload_shared_mib"]
    assert naive_mib == g["unique_payload_naive_mib"]
    assert round(100 * (1 - shared_mib / naive_mib), 2) == g["reduction_percent"]


def test_fork_then_tail_cow_hand_derived():
    # P = 4.  A appends 6 tokens -> pages [0, 1] (page 1 holds 2 tokens).
    t = pt.PageTable(8, 4)
    a = t.create()
    t.append(a, 6)
    assert t.block_table(a) == [0, 1]
    b = t.fork(a)                       # rc(0) = rc(1) = 2, nothing allocated
    assert t.rc[:2] == [2, 2] and t.n_free == 6
    t.append(b, 1)                      # B writes into shared page 1 -> copy to page 2
    assert t.block_table(b) == [0, 2] and t.rc[:3] == [2, 1, 1]
    t.append(a, 1)                      # page 1 now exclusive to A -> written in place
    assert t.block_table(a) == [0, 1]
    t.append(a, 2)                      # token 7 -> page 1 slot 3, token 8 -> new page 3
    assert t.block_table(a) == [0, 1, 3]
    assert list(t.positions(a)) == list(range(9)) and t.info(a) == (9, 9, 3)
    t.check_invariants()


def test_drop_and_repos_hand_derived():
    t = pt.PageTable(8, 4, 1, 2, with_data=True, rope_theta=10.0)
    a = t.create()
    k = np.arange(20, dtype=float).reshape(10, 1, 2)
    t.append(a, 10, k, -k)              # pages [0, 1, 2]
    kept = t.drop(a, [(1, 2)])          # drop tokens 1, 2
    assert list(kept) == [0, 3, 4, 5, 6, 7, 8, 9]
    assert t.block_table(a) == [0, 1] and t.rc[2] == 0 and t.n_free == 6
    assert list(t.positions(a)) == [0, 3, 4, 5, 6, 7, 8, 9] and t.info(a) == (8, 10, 2)
    kk, vv = t.materialise(a)
    assert np.array_equal(vv[:, 0, :], -k[kept, 0, :])   # values moved bit-exactly
    assert np.array_equal(kk[:, 0, :], k[kept, 0, :])    # drop alone does not rotate
    kept2 = t.repos(a)
    assert list(kept2) == list(range(8))
    assert list(t.positions(a)) == list(range(8)) and t.info(a) == (8, 8, 2)
    kk2, vv2 = t.materialise(a)
    delta = np.arange(8) - np.array([0, 3, 4, 5, 6, 7, 8, 9])
    # d = 2: one pair (x0, x1) rotated by delta * theta^0 = delta radians
    c, s = np.cos(delta), np.sin(delta)
    exp = np.stack([kk[:, 0, 0] * c - kk[:, 0, 1] * s, kk[:, 0, 1] * c + kk[:, 0, 0] * s], 1)
    assert np.allclose(kk2[:, 0, :], exp, rtol=0, atol=1e-12)
    assert np.array_equal(vv2, vv)


def test_drop_on_shared_pages_copies_before_freeing():
    t = pt.PageTable(8, 4)
    a = t.create()
    t.append(a, 12)                      # [0, 1, 2]
    b = t.fork(a)
    kept = t.drop(b, [(0, 1)])           # every kept token shifts by one
    assert len(kept) == 11
    # affected logical pages 0, 1, 2 are shared -> copies 3, 4, 5 (allocated before the
    # release of anything); nothing is released since ceil(11/4) = 3
    assert t.block_table(b) == [3, 4, 5] and t.block_table(a) == [0, 1, 2]
    assert t.rc[:6] == [1, 1, 1, 1, 1, 1]
    c = t.fork(a)
    t.drop(c, [(8, 4)])                  # only the tail is dropped: no slot changes
    assert t.block_table(c) == [0, 1] and t.rc[2] == 1
    t.check_invariants()


def test_mount_snapshot_and_cow():
    t = pt.PageTable(16, 4)
    a, b = t.create(), t.create()
    t.append(a, 6)                       # a: [0, 1]
    t.append(b, 3)                       # b: [2]
    t.mount(b, a, 2, 4)                  # tokens 2..5 -> pages 0 and 1 touched
    assert t.rc[:3] == [2, 2, 1]
    t.append(a, 1)                       # page 1 is mounted -> a copies it to page 3
    assert t.block_table(a) == [0, 3]
    assert t.rc[:4] == [2, 1, 1, 1]
    t.release(a)
    assert t.rc[:4] == [1, 1, 1, 0]      # mounted pages survive the release
    t.check_invariants()


def test_rewind_and_oom_leave_state():
    t = pt.PageTable(3, 4)
    a = t.create()
    t.append(a, 9)                       # [0, 1, 2], full pool
    before = (t.block_table(a), list(t.rc), t.n_free, t.info(a))
    with pytest.raises(pt.OOM):
        t.append(a, 4)
    assert (t.block_table(a), list(t.rc), t.n_free, t.info(a)) == before
    t.rewind(a, 5)
    assert t.block_table(a) == [0, 1] and t.n_free == 1 and t.info(a) == (5, 5, 2)
    b = t.fork(a)
    with pytest.raises(pt.OOM):          # b's tail copy + a new page > 1 free page
        t.append(b, 4)
    t.append(b, 3)                       # copy page 1 -> page 2, fits in the tail
    assert t.block_table(b) == [0, 2]
    with pytest.raises(pt.Invalid):
        t.rewind(b, 9)
    t.check_invariants()


# ------------------------------------------------------------------ random op sequences

class Naive:
    """Visible context per sequence as plain lists of (k, v, pos) -- no pages at all."""

    def __init__(self, theta):
        self.own, self.mnt, self.next = [], [], []
        self.theta = theta

    def create(self):
        self.own.append([]); self.mnt.append([]); self.next.append(0)

    def fork(self, p):
        self.own.append(list(self.own[p])); self.mnt.append(list(self.mnt[p]))
        self.next.append(self.next[p])

    def append(self, s, k, v):
        for i in range(len(k)):
            self.own[s].append((k[i], v[i], self.next[s]))
            self.next[s] += 1

    def write(self, s, start, k, v):
        for i in range(len(k)):
            _, _, p = self.own[s][start + i]
            self.own[s][start + i] = (k[i], v[i], p)

    def mount(self, d, s, b, n):
        self.mnt[d] = self.mnt[d] + list(self.own[s][b:b + n])

    def drop(self, s, spans, repos):
        gone = set()
        for b, L in spans:
            gone.update(range(b, b + L))
        kept = [x for i, x in enumerate(self.own[s]) if i not in gone]
        if repos:
            kept = [(rope.rotate(k[None], [j - p], self.theta)[0], v, j) for j, (k, v, p) in enumerate(kept)]
            self.next[s] = len(kept)
        self.own[s] = kept

    def rewind(self, s, n):
        if n != len(self.own[s]):
            self.own[s] = self.own[s][:n]
            self.next[s] = self.own[s][-1][2] + 1 if n else 0

    def visible(self, s):
        return self.own[s] + self.mnt[s]


ops_strategy = st.lists(st.tuples(st.sampled_from(["append", "fork", "mount", "drop", "repos", "rewind",
                                                   "release", "write", "create"]),
                                  st.integers(0, 10**6), st.integers(0, 10**6), st.integers(0, 10**6)),
                        min_size=1, max_size=25)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(ops=ops_strategy, page=st.integers(1, 4), cap=st.integers(2, 16))
def test_random_ops_against_page_free_model(ops, page, cap):
    hkv, d, theta = 1, 4, 100.0
    t = pt.PageTable(cap, page, hkv, d, with_data=True, rope_theta=theta)
    nv = Naive(theta)
    rng = np.random.default_rng(len(ops) * 31 + page)
    t.create(); nv.create()
    for kind, x, y, z in ops:
        live = [i for i, s in enumerate(t.seqs) if s.live]
        snap = {p: (t.kdata[p].copy(), t.vdata[p].copy()) for p in range(cap) if t.rc[p] > 1}
        state = (list(t.rc), t.n_free, [(s.live, list(s.pages), s.n) for s in t.seqs])
        try:
            if kind == "create":
                t.create(); nv.create()
            elif not live:
                continue
            else:
                s = live[x % len(live)]
                n_s = t.seqs[s].n
                if kind == "append":
                    n = y % 7
                    k = rng.standard_normal((n, hkv, d)); v = rng.standard_normal((n, hkv, d))
                    free0 = t.n_free
                    t.append(s, n, k, v); nv.append(s, k, v)
                elif kind == "fork":
                    free0 = t.n_free
                    t.fork(s); nv.fork(s)
                    assert t.n_free == free0
                elif kind == "write" and n_s:
                    a = y % n_s; n = 1 + z % (n_s - a)
                    k = rng.standard_normal((n, hkv, d)); v = rng.standard_normal((n, hkv, d))
                    t.write(s, a, n, k, v); nv.write(s, a, k, v)
                elif kind == "mount" and live:
                    src = live[y % len(live)]
                    ns = t.seqs[src].n
                    if ns:
                        b = z % ns; n = 1 + (x // 7) % (ns - b)
                        t.mount(s, src, b, n); nv.mount(s, src, b, n)
                elif kind in ("drop", "repos"):
                    spans = []
                    if kind == "drop" and n_s:
                        for j in range(y % 3):
                            b = (z * (j + 3)) % n_s
                            spans.append((b, min(n_s - b, 1 + (x + j) % 5)))
                    kept = t.drop(s, spans, repos=(kind == "repos" or z % 2 == 1))
                    nv.drop(s, spans, repos=(kind == "repos" or z % 2 == 1))
                    assert len(kept) == t.seqs[s].n
                elif kind == "rewind":
                    n = y % (n_s + 1)
                    t.rewind(s, n); nv.rewind(s, n)
                elif kind == "release":
                    t.release(s)
        except pt.OOM:
            # a failing call leaves everything unchanged
            assert state == (list(t.rc), t.n_free, [(s.live, list(s.pages), s.n) for s in t.seqs])
            continue
        t.check_invariants()
        for p, (kd, vd) in snap.items():      # a page shared before the op was not written
            if t.rc[p] > 0:
                assert np.array_equal(t.kdata[p], kd) and np.array_equal(t.vdata[p], vd)
        for i, s in enumerate(t.seqs):
            if not s.live:
                continue
            vis = nv.visible(i)
            k, v = t.materialise(i)
            assert k.shape[0] == len(vis)
            if vis:
                assert np.allclose(k, np.stack([a for a, _, _ in vis]), atol=1e-12, rtol=0)
                assert np.array_equal(v, np.stack([b for _, b, _ in vis]))
            assert list(t.positions(i)) == [p for _, _, p in nv.own[i]]
            assert t.info(i)[1] == nv.next[i]
