"""Gradients of the packed DAG prefill (fp64).  Test infrastructure: only the tests, the
smoke check and the bench's CPU baseline use this module.

Octopus (zicq.com page), "Packed DAG-GRPO": the packed episode is trained with one
block-sparse attention whose mask encodes the DAG; the same mask governs the backward
pass, so only DAG-visible (query, key) pairs carry gradient.  The page names the
training throughput, not the gradient formulas; those below are the plain derivative of
softmax attention, written per visible pair from the token-level rule in
oracle/prefill.py (never from a block list).

For query head h (KV head g = h // G), scale c, and a visible pair (i, j):
  s_ij = c q_i.k_j;  P_ij = exp(s_ij - lse_i);  o_i = sum_j P_ij v_j;
  D_i = do_i . o_i;  dP_ij = do_i . v_j;  dS_ij = P_ij (dP_ij - D_i);
  dq_i = c sum_j dS_ij k_j;  dk_j = c sum_{h in g} sum_i dS_ij q_i;
  dv_j = sum_{h in g} sum_i P_ij do_i.
Reading: o_i and lse_i are the oracle's own fp64 forward values (the library takes the
caller's forward outputs instead; they differ by the forward's rounding).

The `magnitudes` forms return, beside each gradient, the same sums taken over the
magnitudes of their terms, |dS_ij| + P_ij d_i with d_i = sum_d |do_i o_i| for dq and dk
and P_ij for dv: a rounding of relative size u in every term of a gradient's sum (or in
D_i) moves it by at most u times that magnitude.
"""
from __future__ import annotations

import numpy as np

from oracle.prefill import _segment_of, visible_mask_row


def _row(q, k, v, do, segments, edges, scale, i, seg_of):
    """Per-row quantities for query i over its visible keys: (idx, P [Hq, n], dS [Hq, n],
    W [Hq, n] = |dS| + P sum_d |do_i o_i|)."""
    T, hq, d = q.shape
    g = hq // k.shape[1]
    idx = np.nonzero(visible_mask_row(segments, edges, T, int(i), seg_of))[0]
    P = np.zeros((hq, len(idx)))
    dS = np.zeros((hq, len(idx)))
    W = np.zeros((hq, len(idx)))
    for h in range(hq):
        kk, vv = k[idx, h // g, :], v[idx, h // g, :]
        s = scale * (kk @ q[i, h])
        m = s.max()
        e = np.exp(s - m)
        p = e / e.sum()
        o = p @ vv
        dp = vv @ do[i, h]
        P[h] = p
        dS[h] = p * (dp - float(do[i, h] @ o))
        W[h] = np.abs(dS[h]) + p * float(np.abs(do[i, h] * o).sum())
    return idx, P, dS, W


def grads(q, k, v, do, segments, edges, scale: float, magnitudes: bool = False):
    """Full gradients (small T): q [T, Hq, d], k/v [T, Hkv, d], do [T, Hq, d] (fp64) ->
    dq [T, Hq, d], dk [T, Hkv, d], dv [T, Hkv, d] (then their magnitudes, if asked)."""
    T, hq, d = q.shape
    g = hq // k.shape[1]
    seg_of = _segment_of(segments, T)
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    mq, mk, mv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for i in range(T):
        idx, P, dS, W = _row(q, k, v, do, segments, edges, scale, i, seg_of)
        for h in range(hq):
            dq[i, h] = scale * (dS[h] @ k[idx, h // g, :])
            dk[idx, h // g, :] += scale * np.outer(dS[h], q[i, h])
            dv[idx, h // g, :] += np.outer(P[h], do[i, h])
            if magnitudes:
                mq[i, h] = scale * (W[h] @ np.abs(k[idx, h // g, :]))
                mk[idx, h // g, :] += scale * np.outer(W[h], np.abs(q[i, h]))
                mv[idx, h // g, :] += np.outer(P[h], np.abs(do[i, h]))
    return (dq, dk, dv, mq, mk, mv) if magnitudes else (dq, dk, dv)


def dq_rows(q, k, v, do, segments, edges, scale: float, rows):
    """dq for the listed query rows only -> ([len(rows), Hq, d], its magnitudes)."""
    T, hq, d = q.shape
    g = hq // k.shape[1]
    seg_of = _segment_of(segments, T)
    out = np.zeros((len(rows), hq, d))
    mag = np.zeros((len(rows), hq, d))
    for r, i in enumerate(rows):
        idx, _, dS, W = _row(q, k, v, do, segments, edges, scale, i, seg_of)
        for h in range(hq):
            out[r, h] = scale * (dS[h] @ k[idx, h // g, :])
            mag[r, h] = scale * (W[h] @ np.abs(k[idx, h // g, :]))
    return out, mag


def seen_by(segments, edges, T: int, j: int) -> np.ndarray:
    """Query indices whose visible set holds key j, from the rule read the other way: the
    later tokens of j's own segment, every token of a segment descending from it, and
    every token of a segment that an edge covering j targets."""
    seg_of = _segment_of(segments, T)
    s = int(seg_of[j])
    parent = [int(p) for _, _, p in segments]

    def descends(t):  # t is a strict descendant of s
        p = parent[t]
        while p >= 0:
            if p == s:
                return True
            p = parent[p]
        return False

    out = [np.arange(j, int(segments[s][0]) + int(segments[s][1]))]
    for t, (st, ln, _p) in enumerate(segments):
        covered = descends(t) or any(
            int(src) == s and int(dst) == t and int(segments[s][0]) + int(off) <= j < int(segments[s][0]) + int(off) + int(ln)
            for src, off, ln, dst in edges)
        if covered:
            out.append(np.arange(int(st), int(st) + int(ln)))
    return np.unique(np.concatenate(out))


def dkdv_keys(q, k, v, do, segments, edges, scale: float, keys):
    """dk, dv for the listed keys only -> [len(keys), Hkv, d] each, then their magnitudes;
    each key's gradient sums over the queries that see it, with each such row's full
    softmax."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    seg_of = _segment_of(segments, T)
    dk, dv, mk, mv = (np.zeros((len(keys), hkv, d)) for _ in range(4))
    rows = {}
    for r, j in enumerate(keys):
        for i in seen_by(segments, edges, T, int(j)):
            if i not in rows:
                rows[i] = _row(q, k, v, do, segments, edges, scale, i, seg_of)
            idx, P, dS, W = rows[i]
            pos = int(np.searchsorted(idx, j))
            for h in range(hq):
                dk[r, h // g] += scale * dS[h, pos] * q[i, h]
                dv[r, h // g] += P[h, pos] * do[i, h]
                mk[r, h // g] += scale * W[h, pos] * np.abs(q[i, h])
                mv[r, h // g] += P[h, pos] * np.abs(do[i, h])
    return dk, dv, mk, mv
