"""Flat page-table oracle: the definition of block tables, refcounts and compaction.

Sources (page / section):
  * Octopus (zicq.com page), "Zero-Copy Radix Forking": a fork adds only a cursor and
    a little metadata and never copies the prefix tensor; KV capacity grows only with
    new tokens; branches share the same physical pages read-only and their own writes
    go to newly allocated pages; writing a shared page in place is forbidden because
    it would corrupt older snapshots.
  * Octopus, "Attention-Only KV Mounting": a thread mounts a sibling's terminal KV
    block with no extra KV allocation.
  * Octopus, core-idea section: the five primitives fork / read_thread / wait_threads
    / rewind / commit.
  * Agentrix (gitlink.org.cn page), "工具数据共享与按需读取" and the cache-lifecycle item:
    local edits create new versions, unchanged pages stay shared, and only blocks
    whose reference count is zero are reclaimed.
  * AKV (news.farwalk.ai page), "AKV 如何工作": Drop removes entries from future
    attention without changing positions; Repos rotates kept keys to positions
    0..r-1 with values unchanged; dropped KV is freed only when no live request
    still needs it.
  * AgentKV (rit.work page): kept entries are physically compacted and the freed
    pages are returned to the allocator.

Readings taken where the pages are silent:
  1. allocation takes the lowest free page id; within one operation copy-on-write
     destinations come first, then new pages in logical order; every allocation of an
     operation happens before any of its frees;
  2. rc(p) = number of (live sequence, logical page) references + number of
     (mount, page) references; p is free iff rc(p) = 0;
  3. fork copies the parent's token count, positions, page list and mounts by
     reference (rc + 1 each) and allocates nothing;
  4. a write to a page with rc > 1 goes to a fresh copy; the writer's reference to
     the old page is dropped;
  5. mount(dst, src, b, n) snapshots tokens [b, b+n) of src's own context (pages
     touched, token offset, positions) and adds one reference to each touched page;
     mounted keys keep src's positions;
  6. drop(spans): spans are half-open token ranges of the own context, unioned;
     kept tokens are packed in order into slots 0..r-1; logical pages before the
     first changed slot keep their ids; affected logical pages below ceil(r/P) are
     rewritten in place when rc = 1, else copied on write; logical pages from
     ceil(r/P) on are released; kept positions and next_pos are unchanged;
     kept_src_idx[j] = old index of the j-th kept token;
  7. repos: kept token j gets position j and next_pos = r; its key is rotated by
     delta_j = j - pos_old(j); values are untouched;
  8. rewind(n) truncates to n tokens, releases pages past ceil(n/P) (the tail page
     stays) and sets next_pos = pos[n-1] + 1 (0 when n = 0); rewinding to the
     current length changes nothing; commit changes nothing;
  9. write(start, n) overwrites tokens in place (positions unchanged), copying every
     touched page whose rc > 1 -- the local edit of an immutable snapshot.
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import rope


class OracleError(Exception):
    pass


class OOM(OracleError):
    pass


class Invalid(OracleError):
    pass


@dataclass
class Mount:
    pages: List[int]
    off: int      # token offset of the first mounted token inside pages[0]
    n: int
    pos: np.ndarray


@dataclass
class Seq:
    pages: List[int] = field(default_factory=list)
    n: int = 0
    pos: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    next_pos: int = 0
    mounts: List[Mount] = field(default_factory=list)
    live: bool = True


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


class PageTable:
    def __init__(self, n_pages: int, page_size: int, n_kv_heads: int = 0, head_dim: int = 0,
                 with_data: bool = False, rope_theta: float = 0.0):
        self.capacity = n_pages
        self.P = page_size
        self.hkv = n_kv_heads
        self.d = head_dim
        self.with_data = with_data
        self.theta = rope_theta
        self.rc = [0] * n_pages
        self._free = list(range(n_pages))  # a sorted list is a valid min-heap
        self.seqs: List[Seq] = []
        self.kdata = {}
        self.vdata = {}

    # ---------------------------------------------------------------- pool primitives
    @property
    def n_free(self) -> int:
        return len(self._free)

    def _alloc(self) -> int:
        p = heapq.heappop(self._free)
        assert self.rc[p] == 0
        self.rc[p] = 1
        if self.with_data:
            self.kdata[p] = np.zeros((self.P, self.hkv, self.d))
            self.vdata[p] = np.zeros((self.P, self.hkv, self.d))
        return p

    def _ref(self, p: int):
        assert self.rc[p] > 0
        self.rc[p] += 1

    def _unref(self, p: int):
        assert self.rc[p] > 0
        self.rc[p] -= 1
        if self.rc[p] == 0:
            heapq.heappush(self._free, p)
            self.kdata.pop(p, None)
            self.vdata.pop(p, None)

    def _seq(self, sid: int) -> Seq:
        if not (0 <= sid < len(self.seqs)) or not self.seqs[sid].live:
            raise Invalid(f"no live sequence {sid}")
        return self.seqs[sid]

    # ---------------------------------------------------------------- primitives
    def create(self) -> int:
        self.seqs.append(Seq())
        return len(self.seqs) - 1

    def fork(self, parent: int) -> int:
        """Reading 3: O(1) in KV bytes, no page allocated."""
        s = self._seq(parent)
        c = Seq(pages=list(s.pages), n=s.n, pos=s.pos.copy(), next_pos=s.next_pos,
                mounts=[Mount(list(m.pages), m.off, m.n, m.pos.copy()) for m in s.mounts])
        for p in c.pages:
            self._ref(p)
        for m in c.mounts:
            for p in m.pages:
                self._ref(p)
        self.seqs.append(c)
        return len(self.seqs) - 1

    def _write(self, sid: int, start: int, n: int, k=None, v=None):
        """Write tokens [start, start+n) of the own context (append when start == s.n)."""
        s = self._seq(sid)
        if n == 0:
            return
        end = start + n
        first, last = start // self.P, (end - 1) // self.P
        cow = [L for L in range(first, min(last + 1, len(s.pages))) if self.rc[s.pages[L]] > 1]
        new = max(0, last + 1 - len(s.pages))
        if len(cow) + new > self.n_free:
            raise OOM(f"need {len(cow) + new} pages, {self.n_free} free")
        for L in cow:  # reading 1: copy-on-write destinations first
            old = s.pages[L]
            p = self._alloc()
            if self.with_data:
                self.kdata[p][:] = self.kdata[old]
                self.vdata[p][:] = self.vdata[old]
            s.pages[L] = p
            self._unref(old)
        for _ in range(new):
            s.pages.append(self._alloc())
        if self.with_data:
            for t in range(n):
                g = start + t
                p = s.pages[g // self.P]
                self.kdata[p][g % self.P] = k[t]
                self.vdata[p][g % self.P] = v[t]

    def append(self, sid: int, n: int, k=None, v=None, pos: Optional[Sequence[int]] = None):
        s = self._seq(sid)
        if n < 0:
            raise Invalid("negative count")
        if pos is None:
            pos = np.arange(s.next_pos, s.next_pos + n, dtype=np.int64)
        pos = np.asarray(pos, np.int64)
        self._write(sid, s.n, n, k, v)
        s.n += n
        s.pos = np.concatenate([s.pos, pos])
        if n:
            s.next_pos = int(pos[-1]) + 1

    def write(self, sid: int, start: int, n: int, k=None, v=None):
        """Reading 9: in-place overwrite of existing tokens (copy-on-write when shared)."""
        s = self._seq(sid)
        if start < 0 or n < 0 or start + n > s.n:
            raise Invalid("write range outside the sequence")
        self._write(sid, start, n, k, v)

    def mount(self, dst: int, src: int, begin: int, n: int):
        """Reading 5."""
        d = self._seq(dst)
        s = self._seq(src)
        if n <= 0 or begin < 0 or begin + n > s.n:
            raise Invalid("mount range outside the source")
        pages = s.pages[begin // self.P: (begin + n - 1) // self.P + 1]
        for p in pages:
            self._ref(p)
        d.mounts.append(Mount(list(pages), begin % self.P, n, s.pos[begin:begin + n].copy()))

    def drop(self, sid: int, spans: Sequence[Tuple[int, int]], repos: bool = False) -> np.ndarray:
        """Readings 6 and 7.  Returns kept_src_idx."""
        s = self._seq(sid)
        dropped = np.zeros(s.n, bool)
        for b, L in spans:
            if b < 0 or L < 0 or b + L > s.n:
                raise Invalid("span outside the sequence")
            dropped[b:b + L] = True
        kept = np.nonzero(~dropped)[0].astype(np.int64)
        r = len(kept)
        old_pos = s.pos[kept]
        new_pos = np.arange(r, dtype=np.int64) if repos else old_pos.copy()
        changed = (kept != np.arange(r)) | (new_pos != old_pos)
        c = int(np.argmax(changed)) if changed.any() else r
        first, n_new = c // self.P, _ceil(r, self.P)
        affected = list(range(first, n_new)) if c < r else []
        cow = [L for L in affected if self.rc[s.pages[L]] > 1]
        if len(cow) > self.n_free:
            raise OOM(f"need {len(cow)} pages, {self.n_free} free")
        if self.with_data:
            k_old, v_old = self._own(s)
            k_new = k_old[kept]
            if repos:
                k_new = rope.rotate(k_new, new_pos - old_pos, self.theta)
            v_new = v_old[kept]
        for L in cow:  # allocations before frees (reading 1)
            old = s.pages[L]
            s.pages[L] = self._alloc()
            self._unref(old)
        for p in s.pages[n_new:]:
            self._unref(p)
        del s.pages[n_new:]
        if self.with_data:
            for j in range(first * self.P, r):
                p = s.pages[j // self.P]
                self.kdata[p][j % self.P] = k_new[j]
                self.vdata[p][j % self.P] = v_new[j]
        s.n = r
        s.pos = new_pos
        if repos:
            s.next_pos = r
        return kept

    def repos(self, sid: int) -> np.ndarray:
        return self.drop(sid, [], repos=True)

    def rewind(self, sid: int, n: int):
        """Reading 8."""
        s = self._seq(sid)
        if n < 0 or n > s.n:
            raise Invalid("rewind beyond the sequence")
        if n == s.n:
            return
        keep = _ceil(n, self.P)
        for p in s.pages[keep:]:
            self._unref(p)
        del s.pages[keep:]
        s.pos = s.pos[:n].copy()
        s.n = n
        s.next_pos = int(s.pos[-1]) + 1 if n else 0

    def commit(self, sid: int):
        self._seq(sid)

    def release(self, sid: int):
        s = self._seq(sid)
        for p in s.pages:
            self._unref(p)
        for m in s.mounts:
            for p in m.pages:
                self._unref(p)
        s.pages, s.mounts, s.live = [], [], False

    # ---------------------------------------------------------------- introspection
    def block_table(self, sid: int) -> List[int]:
        return list(self._seq(sid).pages)

    def positions(self, sid: int) -> np.ndarray:
        return self._seq(sid).pos.copy()

    def info(self, sid: int):
        s = self._seq(sid)
        return s.n, s.next_pos, len(s.pages)

    def check_invariants(self):
        refs = np.zeros(self.capacity, np.int64)
        for s in self.seqs:
            if not s.live:
                continue
            assert len(s.pages) == _ceil(s.n, self.P)
            assert len(s.pos) == s.n
            for p in s.pages:
                refs[p] += 1
            for m in s.mounts:
                for p in m.pages:
                    refs[p] += 1
        assert list(refs) == self.rc, "refcount != number of references"
        assert self.n_free + sum(1 for x in self.rc if x > 0) == self.capacity
        assert sorted(self._free) == [p for p in range(self.capacity) if self.rc[p] == 0]

    # ---------------------------------------------------------------- materialisation
    def _own(self, s: Seq):
        k = np.zeros((s.n, self.hkv, self.d))
        v = np.zeros((s.n, self.hkv, self.d))
        for L, p in enumerate(s.pages):
            a, b = L * self.P, min(s.n, (L + 1) * self.P)
            k[a:b] = self.kdata[p][:b - a]
            v[a:b] = self.vdata[p][:b - a]
        return k, v

    def materialise(self, sid: int):
        """Copy the sequence's whole visible context (own tokens, then mounts) out of the
        pool into contiguous fp64 arrays [n_ctx, Hkv, d]."""
        s = self._seq(sid)
        ks, vs = [], []
        k, v = self._own(s)
        ks.append(k)
        vs.append(v)
        for m in s.mounts:
            for t in range(m.n):
                g = m.off + t
                p = m.pages[g // self.P]
                ks.append(self.kdata[p][g % self.P][None])
                vs.append(self.vdata[p][g % self.P][None])
        return np.concatenate(ks), np.concatenate(vs)


def replay(scenario, with_data: bool = True, to_f64=None) -> Tuple[PageTable, List]:
    """Run a ``workloads.Scenario`` op list on a fresh oracle table.  `to_f64` converts the
    scenario's stored arrays to fp64.  Returns (table, kept_src_idx per drop op)."""
    t = PageTable(scenario.n_pages, scenario.page_size, scenario.n_kv_heads, scenario.head_dim,
                  with_data=with_data, rope_theta=scenario.rope_theta)
    drops = []
    for op in scenario.ops:
        kind = op[0]
        if kind == "create":
            t.create()
        elif kind == "append":
            blk = scenario.blocks[op[2]]
            n = blk.pos.shape[0]
            if with_data:
                t.append(op[1], n, to_f64(blk.k), to_f64(blk.v), blk.pos)
            else:
                t.append(op[1], n, pos=blk.pos)
        elif kind == "fork":
            t.fork(op[1])
        elif kind == "mount":
            t.mount(op[1], op[2], op[3], op[4])
        elif kind == "drop":
            drops.append(t.drop(op[1], op[2], op[3]))
        elif kind == "release":
            t.release(op[1])
        else:
            raise ValueError(kind)
    return t, drops
