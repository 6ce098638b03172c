"""Seeded synthetic workloads for shared-prefix fork / DAG attention.

This module only *draws inputs*. It holds none of the attention, page-table,
drop/compaction or mask arithmetic: the CPU oracle (``oracle/``) and the HIP
path (``fork_attention_decode_amd``) both consume the arrays produced here and
share nothing else.

Shapes and structure follow the five workloads the method is measured on:

* tiny fork decode (fp32, 4q/1kv heads, d=64, 256-token prefix, 4 branches x 64)
* shared-prefix fork decode (bf16, 32q/8kv, d=128, 32K prefix, 16 branches x 2K)
* Octopus-style KV DAG decode (65,536-token root, 8 threads x 8,192, each thread
  mounts the terminal 4,096-token block of 2 siblings)
* AKV-style drop + repos (16 requests x 131,072 tokens, 40% dropped as spans of
  2,048..8,192 tokens, kept keys re-rotated to 0..r-1) then decode
* packed DAG-GRPO prefill (16,384-token prefix + 8 branches x 8,192, 12 cross-branch
  read edges of 2,048 tokens)

Recipe (applies to every generator):
  * ``numpy.random.default_rng(SeedSequence([config_id, purpose, seed]))``;
  * draws are fp64; Q and V ~ N(0, 1); K ~ N(0, 1) / sqrt(d) with softmax scale 1
    (the tiny fp32 case keeps K ~ N(0, 1) unscaled with softmax scale 1/sqrt(d));
  * rotary embedding (NeoX half-split, theta = 1e6) is applied to K and Q at their
    true positions in fp64, then each value is rounded once to the storage type
    (bf16 round-to-nearest-even; fp32 for the tiny case).

bf16 tensors are stored as ``uint16`` bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

# --------------------------------------------------------------------------------------
# storage conversion (input synthesis only)
# --------------------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (round-to-nearest-even) and return the uint16 bits.

    Rounds directly from fp64 (no fp32 double rounding) on the integer image of the
    fp64 value: bf16 keeps the top 7 of fp64's 52 fraction bits, so adding
    2^44 - 1 plus the lowest kept bit and clearing the 45 low bits is an exact
    round-half-even (a carry moves into the exponent as it should).  The result is
    a bf16 value, so its fp32 conversion is exact.  Inputs are N(0,1) draws, far
    from the bf16 overflow and subnormal ranges.
    """
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    u = (u + (np.uint64((1 << 44) - 1) + ((u >> np.uint64(45)) & np.uint64(1)))) & ~np.uint64((1 << 45) - 1)
    return (u.view(np.float64).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32).astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)


def _rng(config_id: int, purpose: int, seed: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([config_id, purpose, seed, sub]))


def _rotate_neox(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Input recipe: rotate fp64 vectors x[n, H, d] at integer positions pos[n]
    (NeoX half-split pairs (i, i + d/2), frequency theta^(-2i/d))."""
    d = x.shape[-1]
    assert d % 2 == 0, "rotary embedding needs an even head dimension"
    half = d // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# purposes (second SeedSequence word)
P_K, P_V, P_Q, P_MOUNT, P_SPANS, P_EDGES, P_DECODE_K, P_DECODE_V = range(8)


# --------------------------------------------------------------------------------------
# decode scenarios
# --------------------------------------------------------------------------------------

@dataclass
class TokenBlock:
    """New tokens for one append: k, v in storage dtype [n, Hkv, d]; pos int64 [n]."""
    k: np.ndarray
    v: np.ndarray
    pos: np.ndarray
    raw_k: Optional[np.ndarray] = None  # fp64 pre-rotation, pre-scale draws (kept only on request)


@dataclass
class Scenario:
    """A sequence of page-table operations followed by one decode query per listed
    sequence.  Sequence ids are assigned in creation order (create / fork), 0, 1, ...

    ops:
      ("create",)                          -> new id
      ("append", sid, block_index)
      ("fork", parent)                     -> new id
      ("mount", dst, src, begin, length)
      ("drop", sid, [(begin, length), ...], repos: bool)
      ("release", sid)
    """
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    sm_scale: float
    rope_theta: float
    n_pages: int
    ops: List[tuple] = field(default_factory=list)
    blocks: List[TokenBlock] = field(default_factory=list)
    queries: List[int] = field(default_factory=list)
    q: Optional[np.ndarray] = None  # [n_queries, Hq, d] storage dtype

    @property
    def n_branches(self) -> int:
        return len(self.queries)


_CHUNK = 16384  # tokens per generation chunk (bounds the fp64 transients)


def _tokens(cid: int, purpose_k: int, purpose_v: int, seed: int, sub: int, n: int, hkv: int, d: int,
            pos: np.ndarray, dtype: str, rope_theta: Optional[float], k_scale: float,
            keep_raw: bool = False) -> TokenBlock:
    """n tokens of one append.  Drawn in chunks: consecutive draws from one generator
    continue its stream, so the values equal one draw of shape (n, hkv, d)."""
    gk = _rng(cid, purpose_k, seed, sub)
    gv = _rng(cid, purpose_v, seed, sub)
    sdt = np.uint16 if dtype == "bf16" else np.float32
    k = np.empty((n, hkv, d), sdt)
    v = np.empty((n, hkv, d), sdt)
    raw = np.empty((n, hkv, d)) if keep_raw else None
    for a in range(0, n, _CHUNK):
        b = min(n, a + _CHUNK)
        xk = gk.standard_normal((b - a, hkv, d))
        if keep_raw:
            raw[a:b] = xk
        kk = _rotate_neox(xk, pos[a:b], rope_theta) if rope_theta else xk
        k[a:b] = _store(kk * k_scale, dtype)
        v[a:b] = _store(gv.standard_normal((b - a, hkv, d)), dtype)
    return TokenBlock(k=k, v=v, pos=pos.astype(np.int64), raw_k=raw)


def _parallel(fn, args_list):
    """Map fn over independent generation jobs on threads (numpy's draws and ufuncs
    release the GIL); results in job order, so values do not depend on scheduling."""
    if len(args_list) <= 1:
        return [fn(*a) for a in args_list]
    with ThreadPoolExecutor(max_workers=min(8, len(args_list), os.cpu_count() or 1)) as ex:
        return list(ex.map(lambda a: fn(*a), args_list))


def _queries(cid: int, seed: int, nq: int, hq: int, d: int, qpos: np.ndarray, dtype: str,
             rope_theta: Optional[float]) -> np.ndarray:
    x = _rng(cid, P_Q, seed).standard_normal((nq, hq, d))
    if rope_theta:
        x = _rotate_neox(x, qpos, rope_theta)
    return _store(x, dtype)


def fork_scenario(prefix: int = 32768, branches: int = 16, private=2048, hq: int = 32, hkv: int = 8,
                  d: int = 128, dtype: str = "bf16", page: int = 16, rope_theta: Optional[float] = 1e6,
                  seed: int = 0, config_id: int = 2, slack_pages: int = 0) -> Scenario:
    """Shared-prefix fork decode: a root appends `prefix` tokens, `branches` forks each
    append their private tokens (the last one is the branch's own decode token), and every
    branch issues one query at the position of its last token.

    `private` may be an int or a per-branch list (ragged branches, empty allowed)."""
    priv = [private] * branches if np.isscalar(private) else list(private)
    assert len(priv) == branches
    scaled = dtype == "bf16"
    k_scale = 1.0 / np.sqrt(d) if scaled else 1.0
    sm_scale = 1.0 if scaled else 1.0 / np.sqrt(d)
    jobs = [(config_id, P_K, P_V, seed, 0, prefix, hkv, d, np.arange(prefix), dtype, rope_theta, k_scale)]
    jobs += [(config_id, P_K, P_V, seed, 1 + b, priv[b], hkv, d, prefix + np.arange(priv[b]), dtype, rope_theta,
              k_scale) for b in range(branches) if priv[b] > 0]
    gen = _parallel(_tokens, jobs)
    blocks = [gen[0]]
    ops: List[tuple] = [("create",), ("append", 0, 0)]
    qpos = []
    for b in range(branches):
        ops.append(("fork", 0))
        sid = 1 + b
        n = priv[b]
        if n > 0:
            blocks.append(gen[len(blocks)])
            ops.append(("append", sid, len(blocks) - 1))
        qpos.append(prefix + max(n, 1) - 1)
    queries = list(range(1, branches + 1))
    q = _queries(config_id, seed, branches, hq, d, np.array(qpos), dtype, rope_theta)
    pages = -(-prefix // page) + sum(-(-n // page) + 1 for n in priv) + slack_pages
    return Scenario(name=f"fork_p{prefix}_b{branches}", n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                    page_size=page, dtype=dtype, sm_scale=sm_scale, rope_theta=rope_theta or 0.0,
                    n_pages=pages, ops=ops, blocks=blocks, queries=queries, q=q)


def dag_scenario(root: int = 65536, threads: int = 8, private: int = 8192, mounts_per_thread: int = 2,
                 mount_len: int = 4096, hq: int = 32, hkv: int = 8, d: int = 128, dtype: str = "bf16",
                 page: int = 16, rope_theta: float = 1e6, seed: int = 0, config_id: int = 3) -> Scenario:
    """Octopus-style KV DAG decode: root prefix, `threads` forks with private tokens, then
    each thread mounts the terminal `mount_len` tokens of `mounts_per_thread` distinct
    seed-chosen siblings (read-only, no copy); one query per thread at its last position."""
    assert mount_len <= private and mounts_per_thread <= threads - 1
    k_scale = 1.0 / np.sqrt(d)
    jobs = [(config_id, P_K, P_V, seed, 0, root, hkv, d, np.arange(root), dtype, rope_theta, k_scale)]
    jobs += [(config_id, P_K, P_V, seed, 1 + t, private, hkv, d, root + np.arange(private), dtype, rope_theta,
              k_scale) for t in range(threads)]
    blocks = _parallel(_tokens, jobs)
    ops: List[tuple] = [("create",), ("append", 0, 0)]
    for t in range(threads):
        ops.append(("fork", 0))
    for t in range(threads):
        ops.append(("append", 1 + t, 1 + t))
    rng = _rng(config_id, P_MOUNT, seed)
    for t in range(threads):
        others = [s for s in range(threads) if s != t]
        pick = rng.choice(len(others), size=mounts_per_thread, replace=False)
        for j in sorted(pick.tolist()):
            s = others[j]
            ops.append(("mount", 1 + t, 1 + s, root + private - mount_len, mount_len))
    queries = list(range(1, threads + 1))
    q = _queries(config_id, seed, threads, hq, d, np.full(threads, root + private - 1), dtype, rope_theta)
    pages = -(-root // page) + threads * (-(-private // page) + 1)
    return Scenario(name=f"dag_r{root}_t{threads}", n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                    page_size=page, dtype=dtype, sm_scale=1.0, rope_theta=rope_theta, n_pages=pages,
                    ops=ops, blocks=blocks, queries=queries, q=q)


def drop_spans(rng: np.random.Generator, n_tokens: int, frac: float, span_min: int, span_max: int
               ) -> List[Tuple[int, int]]:
    """Spans dropping exactly round(frac * n) tokens: lengths ~ U{span_min..span_max}, the last
    one truncated to hit the count; the k+1 kept gaps are a random composition of the kept
    count (sorted uniform cut points; a zero gap joins two spans)."""
    n_drop = int(round(frac * n_tokens))
    lens = []
    tot = 0
    while tot < n_drop:
        L = int(rng.integers(span_min, span_max + 1))
        L = min(L, n_drop - tot)
        lens.append(L)
        tot += L
    kept = n_tokens - n_drop
    cuts = np.sort(rng.integers(0, kept + 1, size=len(lens)))
    gaps = np.diff(np.concatenate([[0], cuts, [kept]]))
    spans = []
    p = int(gaps[0])
    for i, L in enumerate(lens):
        spans.append((p, L))
        p += L + int(gaps[i + 1])
    assert p == n_tokens
    return spans


def drop_scenario(requests: int = 16, ctx: int = 131072, frac: float = 0.4, span_min: int = 2048,
                  span_max: int = 8192, hq: int = 32, hkv: int = 8, d: int = 128, dtype: str = "bf16",
                  page: int = 16, rope_theta: float = 1e6, seed: int = 0, config_id: int = 4,
                  repos: bool = True, keep_raw: bool = False) -> Scenario:
    """AKV-style drop + repos then decode: independent requests append `ctx` tokens, drop
    ~frac of them as contiguous spans (kept keys re-rotated to 0..r-1 when `repos`), then
    append one decode token at position r (or the old next position without repos) and
    issue one query there."""
    k_scale = 1.0 / np.sqrt(d)
    ops: List[tuple] = []
    blocks: List[TokenBlock] = []
    qpos = []
    span_lists = [drop_spans(_rng(config_id, P_SPANS, seed, i), ctx, frac, span_min, span_max)
                  for i in range(requests)]
    dpos = [(ctx - sum(L for _, L in sp)) if repos else ctx for sp in span_lists]
    ctx_blocks = _parallel(_tokens, [(config_id, P_K, P_V, seed, 1 + i, ctx, hkv, d, np.arange(ctx), dtype,
                                      rope_theta, k_scale, keep_raw) for i in range(requests)])
    for i in range(requests):
        ops.append(("create",))
        blocks.append(ctx_blocks[i])
        ops.append(("append", i, len(blocks) - 1))
        ops.append(("drop", i, span_lists[i], repos))
        p = dpos[i]
        blocks.append(_tokens(config_id, P_DECODE_K, P_DECODE_V, seed, 1 + i, 1, hkv, d,
                              np.array([p]), dtype, rope_theta, k_scale, keep_raw=keep_raw))
        ops.append(("append", i, len(blocks) - 1))
        qpos.append(p)
    queries = list(range(requests))
    q = _queries(config_id, seed, requests, hq, d, np.array(qpos), dtype, rope_theta)
    pages = requests * (-(-ctx // page) + 2)
    return Scenario(name=f"drop_n{ctx}_r{requests}", n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                    page_size=page, dtype=dtype, sm_scale=1.0, rope_theta=rope_theta, n_pages=pages,
                    ops=ops, blocks=blocks, queries=queries, q=q)


# --------------------------------------------------------------------------------------
# packed DAG prefill
# --------------------------------------------------------------------------------------

@dataclass
class PrefillInputs:
    """Packed sequence of T tokens.

    segments: int32 [n_seg, 3] rows (start, length, parent) -- segment 0 is the shared
      prefix (parent -1); a segment sees every token of its ancestor segments, its own
      tokens causally, and every edge range that targets it.
    edges: int32 [n_edges, 4] rows (src_segment, src_offset, length, dst_segment).
    q [T, Hq, d], k/v [T, Hkv, d] in storage dtype.
    """
    T: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    sm_scale: float
    block: int
    segments: np.ndarray
    edges: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    pos: np.ndarray


def prefill_inputs(prefix: int = 16384, branches: int = 8, branch_len=8192, n_edges: int = 12,
                   edge_len: int = 2048, hq: int = 32, hkv: int = 8, d: int = 128, dtype: str = "bf16",
                   block: int = 64, rope_theta: float = 1e6, seed: int = 0, config_id: int = 5,
                   with_data: bool = True) -> PrefillInputs:
    """Packed DAG-GRPO prefill: prefix then branches packed back to back; `n_edges` distinct
    ordered branch pairs (s < t, s earlier in sync order) each expose a block-aligned
    `edge_len` range of branch s to every query of branch t.  `branch_len` may be a list
    (ragged branches; only the last may end off a block boundary)."""
    blen = [branch_len] * branches if np.isscalar(branch_len) else list(branch_len)
    starts = [0]
    segs = [(0, prefix, -1)]
    p = prefix
    for b in range(branches):
        segs.append((p, blen[b], 0))
        p += blen[b]
    T = p
    pairs = [(s, t) for t in range(branches) for s in range(t)]
    rng = _rng(config_id, P_EDGES, seed)
    n_edges = min(n_edges, len(pairs))
    sel = rng.choice(len(pairs), size=n_edges, replace=False)
    edges = []
    for i in sorted(sel.tolist()):
        s, t = pairs[i]
        L = min(edge_len, blen[s])
        max_off = (blen[s] - L) // block
        off = int(rng.integers(0, max_off + 1)) * block
        edges.append((1 + s, off, L, 1 + t))
    # positions: prefix 0..prefix-1; each branch continues from the prefix end
    pos = np.concatenate([np.arange(prefix)] + [prefix + np.arange(L) for L in blen]).astype(np.int64)
    q = k = v = None
    if with_data:
        k_scale = 1.0 / np.sqrt(d)
        xk = _rng(config_id, P_K, seed).standard_normal((T, hkv, d))
        k = _store(_rotate_neox(xk, pos, rope_theta) * k_scale, dtype)
        del xk
        v = _store(_rng(config_id, P_V, seed).standard_normal((T, hkv, d)), dtype)
        xq = _rng(config_id, P_Q, seed).standard_normal((T, hq, d))
        q = _store(_rotate_neox(xq, pos, rope_theta), dtype)
        del xq
    return PrefillInputs(T=T, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, dtype=dtype, sm_scale=1.0,
                         block=block, segments=np.array(segs, dtype=np.int32).reshape(-1, 3),
                         edges=np.array(edges, dtype=np.int32).reshape(-1, 4), q=q, k=k, v=v, pos=pos)


# --------------------------------------------------------------------------------------
# named workloads (full sizes) and small variants that span several tiles + ragged tails
# --------------------------------------------------------------------------------------

def tiny_fork(seed: int = 0) -> Scenario:
    """1 layer, 4 query heads / 1 KV head, d=64, fp32, page 16; 256-token prefix,
    4 branches x 64 private tokens; no rotary embedding."""
    return fork_scenario(prefix=256, branches=4, private=64, hq=4, hkv=1, d=64, dtype="f32",
                         rope_theta=None, seed=seed, config_id=1)


def shared_prefix_fork(seed: int = 0) -> Scenario:
    return fork_scenario(seed=seed, config_id=2)


def octopus_dag(seed: int = 0) -> Scenario:
    return dag_scenario(seed=seed, config_id=3)


def akv_drop_repos(seed: int = 0, keep_raw: bool = False) -> Scenario:
    return drop_scenario(seed=seed, config_id=4, keep_raw=keep_raw)


def dag_prefill(seed: int = 0, with_data: bool = True) -> PrefillInputs:
    return prefill_inputs(seed=seed, config_id=5, with_data=with_data)


WORKLOADS = {
    "tiny_fork_decode": tiny_fork,
    "shared_prefix_fork_decode": shared_prefix_fork,
    "octopus_dag_decode": octopus_dag,
    "akv_drop_repos_decode": akv_drop_repos,
    "packed_dag_prefill": dag_prefill,
}
