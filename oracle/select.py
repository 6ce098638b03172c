"""Key scoring and keep selection in front of Drop (fp64).  Test infrastructure: only the
tests, the smoke check and the bench's CPU baseline use this module.

AgentKV (rit.work), section "Как AgentKV выбирает и освобождает записи кэша": the system
keeps a queue of recent attention queries for each phase, merges the queues before a
compression, scores every key against the merged set and keeps the entries with the
highest mean attention (32 representative queries in the main experiments); the kept
entries are then compacted physically and the freed pages returned to the allocator.

Readings (the page gives no formula):
  * the caller passes the merged representative set, n_rep query vectors [n_rep, Hq, d]
    already rotated; the phase queues, their sizes and the phase parser are policy
    outside this path;
  * the attention of representative query r, head h, on key t is t's softmax probability
    in that query's attention over the sequence's whole visible context (own tokens, then
    mounts), reading KV head h // (Hq / Hkv), with the given scale;
  * score(t) = the mean of that probability over the n_rep x Hq (query, head) pairs, for
    each of the sequence's own tokens t (mounted tokens are read-only and never dropped);
  * keep = the `budget` own tokens with the highest score, ties to the lower token index;
    the other tokens are dropped as maximal spans of consecutive tokens.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def key_scores(table, sid: int, q_rep: np.ndarray, scale: float) -> np.ndarray:
    """Mean attention of the representative queries on each own token of sequence `sid`
    of an oracle PageTable (with data).  q_rep [n_rep, Hq, d] fp64 -> scores [n_own]."""
    k, _ = table.materialise(sid)  # own tokens first, then mounts
    n_own = table.info(sid)[0]
    n_rep, hq, _ = q_rep.shape
    g = hq // k.shape[1]
    acc = np.zeros(n_own)
    if k.shape[0] == 0 or n_rep == 0:
        return acc
    for r in range(n_rep):
        for h in range(hq):
            s = scale * (k[:, h // g, :] @ np.asarray(q_rep[r, h], np.float64))
            p = np.exp(s - s.max())
            acc += (p / p.sum())[:n_own]
    return acc / (n_rep * hq)


def select_keep(scores: np.ndarray, budget: int) -> np.ndarray:
    """Boolean keep mask: the `budget` highest scores, ties to the lower index."""
    n = len(scores)
    budget = max(0, min(int(budget), n))
    order = sorted(range(n), key=lambda t: (-float(scores[t]), t))
    keep = np.zeros(n, bool)
    keep[order[:budget]] = True
    return keep


def drop_spans(keep: np.ndarray) -> List[Tuple[int, int]]:
    """Maximal runs of dropped tokens as (begin, length)."""
    spans, t, n = [], 0, len(keep)
    while t < n:
        if keep[t]:
            t += 1
            continue
        a = t
        while t < n and not keep[t]:
            t += 1
        spans.append((a, t - a))
    return spans
