"""Decode attention oracle (fp64): materialise, then textbook softmax attention.

Agentrix README (gitlink.org.cn page, section "前缀复用与 ForkAttention" and the CUDA
ForkAttention item under "初赛基础与决赛演进"): branches that decode together split
their context into a public and a private segment by the actual cache pages, reuse
the loaded public K/V for several queries, then merge each branch's results.  What
that computes is, per branch, ordinary attention over the branch's whole visible
context; the oracle computes exactly that definition, by copying every visible K/V
row out of its page pool into a contiguous array first (no sharing, no splitting).

Readings:
  * visible context = the sequence's own tokens in order, then each mount's token
    range (Octopus page, "Attention-Only KV Mounting": a thread reads a sibling's
    terminal KV block directly);
  * grouped-query mapping: query head h reads KV head h // (Hq / Hkv);
  * output O = softmax(scale * K q) V, LSE = natural log of the softmax normaliser
    plus the max;
  * a row with no keys has O = 0 and LSE = -inf.
"""
from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """One query row against n keys.  q [d], k [n, d], v [n, d] -> (o [d], lse)."""
    q = np.asarray(q, np.float64)
    if k.shape[0] == 0:
        return np.zeros(q.shape[-1]), -np.inf
    s = scale * (np.asarray(k, np.float64) @ q)
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ np.asarray(v, np.float64)) / l, m + np.log(l)


def attend_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """q [Hq, d]; k, v [n, Hkv, d] -> (o [Hq, d], lse [Hq]) with head h reading KV head
    h // (Hq / Hkv)."""
    hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    g = hq // hkv
    o = np.zeros((hq, d))
    lse = np.zeros(hq)
    for h in range(hq):
        o[h], lse[h] = attend(q[h], k[:, h // g, :], v[:, h // g, :], scale)
    return o, lse


def partial(q, k, v, scale):
    """Partial softmax state of one query over a key subset: (m, l, o_unnormalised)."""
    if k.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(np.asarray(q).shape[-1])
    s = scale * (np.asarray(k, np.float64) @ np.asarray(q, np.float64))
    m = s.max()
    p = np.exp(s - m)
    return m, p.sum(), p @ np.asarray(v, np.float64)


def merge(parts):
    """Log-sum-exp merge of partial states (m_i, l_i, o_i):
    M = max m_i, L = sum l_i e^(m_i - M), O = sum o_i e^(m_i - M) / L, LSE = M + ln L.
    Empty parts (m = -inf) contribute nothing."""
    parts = [p for p in parts if np.isfinite(p[0])]
    if not parts:
        return None, -np.inf
    M = max(p[0] for p in parts)
    L = sum(p[1] * np.exp(p[0] - M) for p in parts)
    O = sum(p[2] * np.exp(p[0] - M) for p in parts)
    return O / L, M + np.log(L)


def magnitudes(q, k, v, scale: float):
    """Sizes of the terms of one row's attention, for error bars (no new arithmetic of the
    method): a[e] = sum_j pi_j |v_je| with pi the softmax weights, and the largest score
    magnitude s_abs = scale * max_j sum_i |q_i k_ji|.  q [d], k [n, d], v [n, d]."""
    q = np.asarray(q, np.float64)
    if k.shape[0] == 0:
        return np.zeros(q.shape[-1]), 0.0
    k = np.asarray(k, np.float64)
    s = scale * (k @ q)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ np.abs(np.asarray(v, np.float64)), float(abs(scale) * (np.abs(k) @ np.abs(q)).max())


def decode(table, seqs, q: np.ndarray, scale: float, with_magnitudes: bool = False):
    """Decode for every listed sequence of an oracle ``PageTable`` (with data).

    q [n, Hq, d] (fp64) -> (o [n, Hq, d], lse [n, Hq]); with_magnitudes adds the
    ``magnitudes`` of every row: a [n, Hq, d] and s_abs [n, Hq]."""
    n, hq, d = q.shape
    o = np.zeros((n, hq, d))
    lse = np.zeros((n, hq))
    a = np.zeros((n, hq, d))
    s_abs = np.zeros((n, hq))
    for i, sid in enumerate(seqs):
        k, v = table.materialise(sid)
        qi = np.asarray(q[i], np.float64)
        o[i], lse[i] = attend_heads(qi, k, v, scale)
        if with_magnitudes:
            g = hq // k.shape[1]
            for h in range(hq):
                a[i, h], s_abs[i, h] = magnitudes(qi[h], k[:, h // g, :], v[:, h // g, :], scale)
    if with_magnitudes:
        return o, lse, a, s_abs
    return o, lse


def causal_last(table, sid: int, q, scale: float, rows=None, with_magnitudes: bool = False):
    """Attention of the last n own tokens of sequence `sid` (n = q.shape[0]) of an oracle
    ``PageTable`` (with data): token j of the n attends to the own tokens up to and
    including itself, then to the mounts (AKV page, section "AKV 如何工作": segmented
    batch attention restores an evicted or edited state with one prefill, each segment
    keeping its own positions; each token sees what a decode at that token would see).

    q [n, Hq, d] (fp64; anything indexable by row) -> (o [n, Hq, d], lse [n, Hq]), or
    only the listed rows j, in their order, when `rows` is given; with_magnitudes adds
    the rows' ``magnitudes`` (a, s_abs) as in ``decode``."""
    n, hq, d = q.shape
    k, v = table.materialise(sid)  # own tokens, then mounts
    n_own = table.info(sid)[0]
    rows = list(range(n)) if rows is None else [int(j) for j in rows]
    o = np.zeros((len(rows), hq, d))
    lse = np.zeros((len(rows), hq))
    a = np.zeros((len(rows), hq, d))
    s_abs = np.zeros((len(rows), hq))
    g = hq // k.shape[1]
    for r, j in enumerate(rows):
        end = n_own - n + j + 1
        idx = np.concatenate([np.arange(end), np.arange(n_own, k.shape[0])]).astype(np.int64)
        qj = np.asarray(q[j], np.float64)
        o[r], lse[r] = attend_heads(qj, k[idx], v[idx], scale)
        if with_magnitudes:
            for h in range(hq):
                a[r, h], s_abs[r, h] = magnitudes(qj[h], k[idx][:, h // g, :], v[idx][:, h // g, :], scale)
    if with_magnitudes:
        return o, lse, a, s_abs
    return o, lse
