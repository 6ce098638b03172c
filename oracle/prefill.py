"""Packed DAG prefill oracle (fp64).

Octopus (zicq.com page), "Packed DAG-GRPO": all branches of an episode are packed
into one block-sparse attention whose mask encodes causality inside a thread, the
allowed cross-thread read edges and the synchronisation dependencies; only block
pairs the DAG allows are computed (the cost paragraph of that section).

The oracle works at token level from the rule itself, never from a block list:
  * a query in segment S at packed index i sees every token of S's ancestor
    segments, the tokens of S at index <= i, and every edge range whose target
    is S (the edge's source is earlier in sync order, hence complete);
  * attention per row is dense softmax over the visible keys, in fp64.

Block counts (what a block-sparse kernel must visit) are derived from the same
token rule: a (query block, key block) pair is needed iff any of its token pairs
is visible.
"""
from __future__ import annotations

import numpy as np


def _segment_of(segments: np.ndarray, T: int) -> np.ndarray:
    seg = np.full(T, -1, np.int64)
    for sidx, (st, ln, _par) in enumerate(segments):
        seg[st:st + ln] = sidx
    return seg


def visible_ranges(segments: np.ndarray, edges: np.ndarray, sidx: int):
    """Key ranges (start, end) visible to every query of segment `sidx`, excluding the
    segment's own causal part."""
    out = []
    par = int(segments[sidx][2])
    while par >= 0:
        st, ln, pp = (int(x) for x in segments[par])
        out.append((st, st + ln))
        par = pp
    for src, off, ln, dst in edges:
        if int(dst) == sidx:
            st = int(segments[src][0]) + int(off)
            out.append((st, st + int(ln)))
    return out


def visible_mask_row(segments, edges, T: int, i: int, seg_of=None) -> np.ndarray:
    seg_of = _segment_of(segments, T) if seg_of is None else seg_of
    s = int(seg_of[i])
    row = np.zeros(T, bool)
    for a, b in visible_ranges(segments, edges, s):
        row[a:b] = True
    row[int(segments[s][0]):i + 1] = True
    return row


def visible_mask(segments, edges, T: int) -> np.ndarray:
    """Dense token mask [T, T] (small T only)."""
    seg_of = _segment_of(segments, T)
    return np.stack([visible_mask_row(segments, edges, T, i, seg_of) for i in range(T)])


def visible_count(segments, edges, T: int) -> int:
    """Number of visible (query, key) token pairs, counted row by row from the rule."""
    seg_of = _segment_of(segments, T)
    total = 0
    for s, (st, ln, _p) in enumerate(segments):
        row = np.zeros(T, bool)
        for a, b in visible_ranges(segments, edges, s):
            row[a:b] = True
        fixed = int(row[:st].sum() + row[st + ln:].sum())  # ranges never overlap the own part
        total += fixed * int(ln) + int(ln) * (int(ln) + 1) // 2
    return total


def block_pairs(segments, edges, T: int, block: int) -> np.ndarray:
    """Boolean [nb, nb]: query block qb needs key block kb iff some token pair is visible."""
    nb = -(-T // block)
    seg_of = _segment_of(segments, T)
    need = np.zeros((nb, nb), bool)
    for qb in range(nb):
        acc = np.zeros(T, bool)
        for i in range(qb * block, min(T, (qb + 1) * block)):
            acc |= visible_mask_row(segments, edges, T, i, seg_of)
        pad = np.zeros(nb * block, bool)
        pad[:T] = acc
        need[qb] = pad.reshape(nb, block).any(axis=1)
    return need


def attend_rows(q, k, v, segments, edges, rows, scale: float, with_magnitudes: bool = False):
    """Dense masked attention for the listed query rows.

    q [T, Hq, d] (fp64, or anything that yields fp64 rows when indexed), k/v [T, Hkv, d]
    (fp64) -> o [len(rows), Hq, d], lse [len(rows), Hq]; with_magnitudes adds, per row and
    head, a = sum_j pi_j |v_j| [len(rows), Hq, d] and s_abs = scale * max_j sum_i |q_i k_ji|
    [len(rows), Hq] over the visible keys (sizes of the terms, for error bars).

    A row's visible keys are its segment's fixed ranges (ancestors, edge sources) and its
    own segment up to itself; rows of one segment are evaluated together as one masked
    product, key range by key range (every key of a range is read in place)."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    seg_of = _segment_of(segments, T)
    kt = np.ascontiguousarray(np.transpose(k, (1, 0, 2)))  # [Hkv, T, d]
    vt = np.ascontiguousarray(np.transpose(v, (1, 0, 2)))
    rows = [int(i) for i in rows]
    o = np.zeros((len(rows), hq, d))
    lse = np.zeros((len(rows), hq))
    a_out = np.zeros((len(rows), hq, d)) if with_magnitudes else None
    s_out = np.zeros((len(rows), hq)) if with_magnitudes else None
    by_seg = {}
    for r, i in enumerate(rows):
        by_seg.setdefault(int(seg_of[i]), []).append(r)
    for s, rs in by_seg.items():
        st = int(segments[s][0])
        for c0 in range(0, len(rs), 64):  # a group of rows of one segment
            grp = rs[c0:c0 + 64]
            ii = np.array([rows[r] for r in grp])
            ranges = list(visible_ranges(segments, edges, s)) + [(st, int(ii.max()) + 1)]
            qg = np.stack([np.asarray(q[int(i)], np.float64) for i in ii])  # [R, Hq, d]
            for hk in range(hkv):
                qh = qg[:, hk * g:(hk + 1) * g, :].reshape(-1, d)  # [R * G, d]
                parts = [scale * (qh @ kt[hk, a:b].T) for a, b in ranges]
                own = parts[-1].reshape(len(grp), g, -1)
                later = np.arange(st, ranges[-1][1])[None, :] > ii[:, None]  # [R, keys]: key after the query
                own[np.broadcast_to(later[:, None, :], own.shape)] = -np.inf  # causal
                m = np.max([p.max(axis=1) for p in parts], axis=0)  # [R * G]
                ps = [np.exp(p - m[:, None]) for p in parts]
                l = np.sum([p.sum(axis=1) for p in ps], axis=0)
                oh = sum(p @ vt[hk, a:b] for p, (a, b) in zip(ps, ranges)) / l[:, None]
                o[grp, hk * g:(hk + 1) * g] = oh.reshape(len(grp), g, d)
                lse[grp, hk * g:(hk + 1) * g] = (m + np.log(l)).reshape(len(grp), g)
                if with_magnitudes:
                    ah = sum(p @ np.abs(vt[hk, a:b]) for p, (a, b) in zip(ps, ranges)) / l[:, None]
                    a_out[grp, hk * g:(hk + 1) * g] = ah.reshape(len(grp), g, d)
                    sa = []
                    for (a, b), p in zip(ranges, parts):
                        t = abs(scale) * (np.abs(qh) @ np.abs(kt[hk, a:b]).T)
                        t[~np.isfinite(p)] = 0.0  # masked keys are not read
                        sa.append(t.max(axis=1))
                    s_out[grp, hk * g:(hk + 1) * g] = np.max(sa, axis=0).reshape(len(grp), g)
    if with_magnitudes:
        return o, lse, a_out, s_out
    return o, lse
