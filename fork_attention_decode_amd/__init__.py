"""Python binding of libforkattn.so -- attention over a shared, paged KV-state DAG on MI355X.

Argument marshalling only: every step of the hot path runs in the library's HIP kernels
(gfx950).  Functions carry the C ABI's names (see include/forkattn.h); PyTorch is used
for device memory and streams.  Importing this package fails loudly when the library
has not been built (``python fork_attention_decode_amd/build.py``); there is no CPU
fallback.

``Pool`` is a convenience holder of the torch buffers a pool needs.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libforkattn.so")

KV_OK, KV_ERR_INVALID, KV_ERR_OOM, KV_ERR_NOT_FOUND, KV_ERR_HIP, KV_ERR_UNSUPPORTED, KV_ERR_WORKSPACE = (
    0, -1, -2, -3, -4, -5, -6)
KV_BF16, KV_F32 = 0, 1
KV_ROPE_NONE, KV_ROPE_NEOX = 0, 1
KV_DROP_REPOS = 1


class ForkAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {status} ({msg})")
        self.status = status


class kv_pool_config(C.Structure):
    _fields_ = [("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("page_size", C.c_int32),
                ("n_pages", C.c_int32), ("dtype", C.c_int32), ("rope_style", C.c_int32),
                ("rope_theta", C.c_double)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python fork_attention_decode_amd/build.py`")
    # torch ships its own HIP runtime (same soname): load it first so that the library
    # binds to that one runtime instead of bringing a second copy into the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    return C.CDLL(LIB_PATH)


lib = _load()

_P = C.c_void_p
_i32, _i64, _sz = C.c_int32, C.c_int64, C.c_size_t
_pi32, _pi64, _psz = C.POINTER(C.c_int32), C.POINTER(C.c_int64), C.POINTER(C.c_size_t)
_SIGS = {
    "kv_pool_bytes": [C.POINTER(kv_pool_config), _psz],
    "kv_pool_workspace_size": [C.POINTER(kv_pool_config), _psz],
    "kv_pool_create": [C.POINTER(kv_pool_config), _P, _P, _P, _sz, C.POINTER(_P)],
    "kv_pool_destroy": [_P],
    "kv_seq_create": [_P, _pi32],
    "kv_append": [_P, _i32, _i64, _P, _P, _pi64, _P],
    "kv_append_batch": [_P, _pi32, _i32, _P, _P, _P],
    "kv_write": [_P, _i32, _i64, _i64, _P, _P, _P],
    "kv_fork": [_P, _i32, _pi32],
    "kv_mount": [_P, _i32, _i32, _i64, _i64],
    "kv_drop": [_P, _i32, _pi64, _pi64, _i32, _i32, _pi64, _P],
    "kv_drop_batch": [_P, _pi32, _i32, _pi64, _pi64, _pi64, _i32, _pi64, _P],
    "kv_repos": [_P, _i32, _P],
    "kv_rewind": [_P, _i32, _i64],
    "kv_commit": [_P, _i32],
    "kv_release": [_P, _i32],
    "kv_seq_info": [_P, _i32, _pi64, _pi64, _pi32, _pi32],
    "kv_block_table": [_P, _i32, _pi32, _i32],
    "kv_positions": [_P, _i32, _pi64, _i64],
    "kv_page_refcount": [_P, _i32, _pi32],
    "kv_free_pages": [_P, _pi32],
    "kv_pool_read_page": [_P, _i32, _i32, _P, _P, _P],
    "kv_pool_sync_status": [_P, _P, _pi32],
    "kv_pool_set_compute_units": [_P, _i32],
    "kv_probe_stream_read": [_P, _sz, _P, _P],
    "kv_probe_mfma_loop": [_i32, _i32, _P, _P],
    "fork_attn_workspace_size": [_P, _pi32, _i32, _i32, _psz],
    "fork_attn_decode": [_P, _pi32, _i32, _i32, _P, _P, _P, C.c_float, _P, _sz, _P],
    "fork_attn_decode_static": [_P, _pi32, _i32, _i32, _P, _P, _P, C.c_float, _P],
    "fork_attn_plan_stats": [_P, _pi64, _i32],
    "fork_attn_partials": [_P, _pi32, _i32, _i32, _P, C.c_float, _P, _sz, _P],
    "fork_attn_merge": [_P, _pi32, _i32, _i32, _P, _P, _P, _sz, _P],
    "dag_mask_build": [_pi32, _i32, _pi32, _i32, _i32, _i32, _pi32, _pi32, C.POINTER(C.c_uint8), _pi64],
    "dag_attn_workspace_size": [_i32, _i32, _i32, _i32, C.c_int64, _psz],
    "dag_attn_prefill": [_P, _P, _P, _P, _P, _i32, _i32, _i32, _i32, _P, _P, _P, C.c_int64, _i32, C.c_float, _P,
                         _sz, _P],
    "dag_attn_prepare": [_P, _P, _i32, _i32, _i32, _i32, _P, _P, _P, C.c_int64, _i32, _P, _sz, _P],
    "dag_attn_run": [_P, _P, _P, _i32, _i32, _i32, _i32, _P, C.c_int64, _i32, C.c_float, _P, _sz, _P],
    "kv_causal_attend_workspace_size": [_P, _i32, C.c_int64, _i32, _psz],
    "kv_causal_attend": [_P, _i32, C.c_int64, _i32, _P, _P, _P, C.c_float, _P, _sz, _P],
    "kv_window_plan": [_P, _pi32, _i32, _i32, _i32, _psz],
    "kv_window_upload": [_P, _P, _sz, _P],
    "kv_window_step": [_P, _i32, _P, _P, _P, _P, _P, C.c_float, _P],
    "dag_attn_backward_workspace_size": [_i32, _i32, _i32, _i32, C.c_int64, _psz],
    "dag_attn_backward": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _i32, _i32, _i32, _i32, _P, _P, _P, C.c_int64, _i32,
                          C.c_float, _P, _sz, _P],
    "kv_score_workspace_size": [_P, _i32, _i32, _i32, _psz],
    "kv_score": [_P, _i32, _P, _i32, _i32, C.c_float, _P, _P, _sz, _P],
    "kv_select_workspace_size": [C.c_int64, _psz],
    "kv_select_keep": [_P, C.c_int64, C.c_int64, _P, _P, _sz, _P],
    "kv_drop_keep": [_P, _i32, C.POINTER(C.c_uint8), C.c_int64, _i32, _P],
}
EXPORTED = sorted(list(_SIGS) + ["kv_status_str", "kv_last_error"])
for _name, _args in _SIGS.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = C.c_int
lib.kv_status_str.argtypes = [C.c_int]
lib.kv_status_str.restype = C.c_char_p
lib.kv_last_error.argtypes = [_P]
lib.kv_last_error.restype = C.c_char_p


def kv_status_str(status: int) -> str:
    return lib.kv_status_str(status).decode()


def kv_last_error(pool: Optional[int] = None) -> str:
    return lib.kv_last_error(pool).decode()


def _check(fn: str, status: int, pool=None):
    if status != KV_OK:
        raise ForkAttnError(fn, status, f"{kv_status_str(status)}: {kv_last_error(pool)}")


def _i64arr(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(C.POINTER(ct))


# ------------------------------------------------------------------ C ABI, same names
def make_config(n_kv_heads, head_dim, n_pages, dtype=KV_BF16, page_size=16, rope_theta=0.0) -> kv_pool_config:
    return kv_pool_config(n_kv_heads, head_dim, page_size, n_pages, dtype,
                          KV_ROPE_NEOX if rope_theta else KV_ROPE_NONE, float(rope_theta))


def kv_pool_bytes(cfg: kv_pool_config) -> int:
    out = C.c_size_t()
    _check("kv_pool_bytes", lib.kv_pool_bytes(C.byref(cfg), C.byref(out)))
    return out.value


def kv_pool_workspace_size(cfg: kv_pool_config) -> int:
    out = C.c_size_t()
    _check("kv_pool_workspace_size", lib.kv_pool_workspace_size(C.byref(cfg), C.byref(out)))
    return out.value


def kv_pool_create(cfg: kv_pool_config, k_pages: int = 0, v_pages: int = 0, workspace: int = 0,
                   ws_bytes: int = 0) -> int:
    h = C.c_void_p()
    _check("kv_pool_create", lib.kv_pool_create(C.byref(cfg), k_pages or None, v_pages or None,
                                                workspace or None, ws_bytes, C.byref(h)))
    return h.value


def kv_pool_destroy(pool: int):
    _check("kv_pool_destroy", lib.kv_pool_destroy(pool), None)


def kv_seq_create(pool: int) -> int:
    s = C.c_int32()
    _check("kv_seq_create", lib.kv_seq_create(pool, C.byref(s)), pool)
    return s.value


def kv_append(pool: int, seq: int, n: int, k: int = 0, v: int = 0, positions=None, stream: int = 0):
    pos = None if positions is None else _i64arr(positions)
    _check("kv_append", lib.kv_append(pool, seq, n, k or None, v or None,
                                      None if pos is None else _ptr(pos, C.c_int64), stream or None), pool)


def kv_append_batch(pool: int, seqs: Sequence[int], k: int = 0, v: int = 0, stream: int = 0):
    s = np.ascontiguousarray(np.asarray(seqs, np.int32))
    _check("kv_append_batch", lib.kv_append_batch(pool, _ptr(s, C.c_int32), len(s), k or None, v or None,
                                                  stream or None), pool)


def kv_write(pool: int, seq: int, start: int, n: int, k: int = 0, v: int = 0, stream: int = 0):
    _check("kv_write", lib.kv_write(pool, seq, start, n, k or None, v or None, stream or None), pool)


def kv_fork(pool: int, parent: int) -> int:
    s = C.c_int32()
    _check("kv_fork", lib.kv_fork(pool, parent, C.byref(s)), pool)
    return s.value


def kv_mount(pool: int, dst: int, src: int, begin: int, length: int):
    _check("kv_mount", lib.kv_mount(pool, dst, src, begin, length), pool)


def kv_drop(pool: int, seq: int, spans: Sequence[Tuple[int, int]], flags: int = 0, stream: int = 0) -> np.ndarray:
    n_tok = kv_seq_info(pool, seq)[0]
    b = _i64arr([s[0] for s in spans]) if len(spans) else np.zeros(1, np.int64)
    L = _i64arr([s[1] for s in spans]) if len(spans) else np.zeros(1, np.int64)
    kept = np.zeros(max(1, n_tok), np.int64)
    _check("kv_drop", lib.kv_drop(pool, seq, _ptr(b, C.c_int64), _ptr(L, C.c_int64), len(spans), flags,
                                  _ptr(kept, C.c_int64), stream or None), pool)
    return kept[:kv_seq_info(pool, seq)[0]].copy()


def kv_drop_batch(pool: int, seqs: Sequence[int], spans_per_seq, flags: int = 0, stream: int = 0):
    """Drops of several sequences in one call; spans_per_seq[i] = [(begin, len), ...] of
    seqs[i].  Returns the compaction index of each sequence (list of arrays)."""
    s = np.ascontiguousarray(np.asarray(seqs, np.int32))
    n_tok = [kv_seq_info(pool, int(q))[0] for q in s]
    off = np.zeros(len(s) + 1, np.int64)
    for i, sp in enumerate(spans_per_seq):
        off[i + 1] = off[i] + len(sp)
    flat = [x for sp in spans_per_seq for x in sp]
    b = _i64arr([x[0] for x in flat]) if flat else np.zeros(1, np.int64)
    L = _i64arr([x[1] for x in flat]) if flat else np.zeros(1, np.int64)
    kept = np.zeros(max(1, sum(n_tok)), np.int64)
    _check("kv_drop_batch", lib.kv_drop_batch(pool, _ptr(s, C.c_int32), len(s), _ptr(off, C.c_int64),
                                              _ptr(b, C.c_int64), _ptr(L, C.c_int64), flags,
                                              _ptr(kept, C.c_int64), stream or None), pool)
    out, at = [], 0
    for q, n in zip(s, n_tok):
        out.append(kept[at:at + kv_seq_info(pool, int(q))[0]].copy())
        at += n
    return out


def kv_repos(pool: int, seq: int, stream: int = 0):
    _check("kv_repos", lib.kv_repos(pool, seq, stream or None), pool)


def kv_rewind(pool: int, seq: int, new_len: int):
    _check("kv_rewind", lib.kv_rewind(pool, seq, new_len), pool)


def kv_commit(pool: int, seq: int):
    _check("kv_commit", lib.kv_commit(pool, seq), pool)


def kv_release(pool: int, seq: int):
    _check("kv_release", lib.kv_release(pool, seq), pool)


def kv_seq_info(pool: int, seq: int) -> Tuple[int, int, int, int]:
    n, p, np_, nm = C.c_int64(), C.c_int64(), C.c_int32(), C.c_int32()
    _check("kv_seq_info", lib.kv_seq_info(pool, seq, C.byref(n), C.byref(p), C.byref(np_), C.byref(nm)), pool)
    return n.value, p.value, np_.value, nm.value


def kv_block_table(pool: int, seq: int) -> np.ndarray:
    n_pages = kv_seq_info(pool, seq)[2]
    out = np.zeros(max(1, n_pages), np.int32)
    _check("kv_block_table", lib.kv_block_table(pool, seq, _ptr(out, C.c_int32), n_pages), pool)
    return out[:n_pages].copy()


def kv_positions(pool: int, seq: int) -> np.ndarray:
    n = kv_seq_info(pool, seq)[0]
    out = np.zeros(max(1, n), np.int64)
    _check("kv_positions", lib.kv_positions(pool, seq, _ptr(out, C.c_int64), n), pool)
    return out[:n].copy()


def kv_page_refcount(pool: int, page: int) -> int:
    rc = C.c_int32()
    _check("kv_page_refcount", lib.kv_page_refcount(pool, page, C.byref(rc)), pool)
    return rc.value


def kv_free_pages(pool: int) -> int:
    n = C.c_int32()
    _check("kv_free_pages", lib.kv_free_pages(pool, C.byref(n)), pool)
    return n.value


def kv_pool_read_page(pool: int, page: int, head: int, k_out: np.ndarray, v_out: np.ndarray, stream: int = 0):
    _check("kv_pool_read_page", lib.kv_pool_read_page(pool, page, head, k_out.ctypes.data, v_out.ctypes.data,
                                                      stream or None), pool)


def kv_pool_set_compute_units(pool: int, n_cu: int) -> None:
    _check("kv_pool_set_compute_units", lib.kv_pool_set_compute_units(pool, n_cu), pool)


def kv_probe_stream_read(buf: int, nbytes: int, sink: int, stream: int = 0) -> None:
    _check("kv_probe_stream_read", lib.kv_probe_stream_read(buf, nbytes, sink, stream or None), None)


def kv_probe_mfma_loop(n_iter: int, n_workgroups: int, sink: int, stream: int = 0) -> None:
    _check("kv_probe_mfma_loop", lib.kv_probe_mfma_loop(n_iter, n_workgroups, sink, stream or None), None)


def kv_pool_sync_status(pool: int, stream: int = 0) -> int:
    n = C.c_int32()
    _check("kv_pool_sync_status", lib.kv_pool_sync_status(pool, stream or None, C.byref(n)), pool)
    return n.value


def fork_attn_workspace_size(pool: int, seqs: Sequence[int], n_q_heads: int) -> int:
    s = np.ascontiguousarray(np.asarray(seqs, np.int32))
    out = C.c_size_t()
    _check("fork_attn_workspace_size", lib.fork_attn_workspace_size(pool, _ptr(s, C.c_int32), len(s), n_q_heads,
                                                                    C.byref(out)), pool)
    return out.value


def fork_attn_decode(pool: int, seqs: Sequence[int], n_q_heads: int, q: int, out: int, lse: int,
                     sm_scale: float, workspace: int, ws_bytes: int, stream: int = 0):
    s = np.ascontiguousarray(np.asarray(seqs, np.int32))
    _check("fork_attn_decode", lib.fork_attn_decode(pool, _ptr(s, C.c_int32), len(s), n_q_heads, q, out,
                                                    lse or None, sm_scale, workspace, ws_bytes, stream or None),
           pool)


FORKATTN_STATIC_WORKSPACE_BYTES = 32 << 20


def fork_attn_decode_static(pool: int, seqs: Sequence[int], n_q_heads: int, q: int, out: int, lse: int,
                            sm_scale: float, stream: int = 0):
    s = np.ascontiguousarray(np.asarray(seqs, np.int32))
    _check("fork_attn_decode_static", lib.fork_attn_decode_static(pool, _ptr(s, C.c_int32), len(s), n_q_heads, q, out,
                                                                  lse or None, sm_scale, stream or None), pool)


def fork_attn_partials(pool: int, seqs: Sequence[int], n_q_heads: int, q: int, sm_scale: float, workspace: int,
                       ws_bytes: int, stream: int = 0):
    s = np.ascontiguousarray(np.asarray(seqs, np.int32))
    _check("fork_attn_partials", lib.fork_attn_partials(pool, _ptr(s, C.c_int32), len(s), n_q_heads, q, sm_scale,
                                                        workspace, ws_bytes, stream or None), pool)


def fork_attn_merge(pool: int, seqs: Sequence[int], n_q_heads: int, out: int, lse: int, workspace: int,
                    ws_bytes: int, stream: int = 0):
    s = np.ascontiguousarray(np.asarray(seqs, np.int32))
    _check("fork_attn_merge", lib.fork_attn_merge(pool, _ptr(s, C.c_int32), len(s), n_q_heads, out, lse or None,
                                                  workspace, ws_bytes, stream or None), pool)


def kv_score_workspace_size(pool: int, seq: int, n_rep: int, n_q_heads: int) -> int:
    out = C.c_size_t(0)
    _check("kv_score_workspace_size", lib.kv_score_workspace_size(pool, seq, n_rep, n_q_heads, C.byref(out)), pool)
    return out.value


def kv_score(pool: int, seq: int, q_rep: int, n_rep: int, n_q_heads: int, sm_scale: float, scores: int,
             workspace: int, ws_bytes: int, stream: int = 0):
    _check("kv_score", lib.kv_score(pool, seq, q_rep, n_rep, n_q_heads, sm_scale, scores, workspace, ws_bytes,
                                    stream or None), pool)


def kv_select_workspace_size(n: int) -> int:
    out = C.c_size_t(0)
    _check("kv_select_workspace_size", lib.kv_select_workspace_size(n, C.byref(out)))
    return out.value


def kv_select_keep(scores: int, n: int, budget: int, keep: int, workspace: int, ws_bytes: int, stream: int = 0):
    _check("kv_select_keep", lib.kv_select_keep(scores, n, budget, keep, workspace or None, ws_bytes, stream or None))


def kv_drop_keep(pool: int, seq: int, keep: np.ndarray, flags: int = 0, stream: int = 0):
    k = np.ascontiguousarray(np.asarray(keep, np.uint8))
    _check("kv_drop_keep", lib.kv_drop_keep(pool, seq, _ptr(k, C.c_uint8), len(k), flags, stream or None), pool)


def fork_attn_plan_stats(pool: int) -> dict:
    out = np.zeros(8, np.int64)
    _check("fork_attn_plan_stats", lib.fork_attn_plan_stats(pool, _ptr(out, C.c_int64), 8), pool)
    keys = ["segments", "items", "chunks", "partials", "unique_kv_bytes", "rows", "longest_item_chunks",
            "patched_changes"]
    return dict(zip(keys, (int(x) for x in out)))


def dag_mask_build(segments, edges, T: int, block: int = 64):
    seg = np.ascontiguousarray(np.asarray(segments, np.int32).reshape(-1, 3))
    ed = np.ascontiguousarray(np.asarray(edges, np.int32).reshape(-1, 4))
    if ed.size == 0:
        ed = np.zeros((1, 4), np.int32)
    n_edges = 0 if np.asarray(edges).size == 0 else len(ed)
    nb = -(-T // block)
    row_ptr = np.zeros(nb + 1, np.int32)
    nnz = C.c_int64()
    _check("dag_mask_build", lib.dag_mask_build(_ptr(seg, C.c_int32), len(seg), _ptr(ed, C.c_int32), n_edges, T,
                                                block, _ptr(row_ptr, C.c_int32), None, None, C.byref(nnz)))
    col = np.zeros(max(1, nnz.value), np.int32)
    kind = np.zeros(max(1, nnz.value), np.uint8)
    _check("dag_mask_build", lib.dag_mask_build(_ptr(seg, C.c_int32), len(seg), _ptr(ed, C.c_int32), n_edges, T,
                                                block, _ptr(row_ptr, C.c_int32), _ptr(col, C.c_int32),
                                                _ptr(kind, C.c_uint8), C.byref(nnz)))
    return row_ptr, col[:nnz.value].copy(), kind[:nnz.value].copy()


def dag_attn_workspace_size(T: int, n_q_heads: int, n_kv_heads: int, block: int = 64, nnz: int = 0) -> int:
    out = C.c_size_t()
    _check("dag_attn_workspace_size", lib.dag_attn_workspace_size(T, n_q_heads, n_kv_heads, block, nnz,
                                                                  C.byref(out)))
    return out.value


def dag_attn_prefill(q: int, k: int, v: int, out: int, lse: int, T: int, n_q_heads: int, n_kv_heads: int,
                     head_dim: int, row_ptr: int, col: int, kind: int, nnz: int, block: int, sm_scale: float,
                     workspace: int, ws_bytes: int, stream: int = 0):
    _check("dag_attn_prefill", lib.dag_attn_prefill(q, k, v, out, lse or None, T, n_q_heads, n_kv_heads, head_dim,
                                                    row_ptr, col, kind, nnz, block, sm_scale, workspace or None,
                                                    ws_bytes, stream or None))


def dag_attn_prepare(k: int, v: int, T: int, n_q_heads: int, n_kv_heads: int, head_dim: int, row_ptr: int, col: int,
                     kind: int, nnz: int, block: int, workspace: int, ws_bytes: int, stream: int = 0):
    _check("dag_attn_prepare", lib.dag_attn_prepare(k, v, T, n_q_heads, n_kv_heads, head_dim, row_ptr, col, kind, nnz,
                                                    block, workspace or None, ws_bytes, stream or None))


def dag_attn_run(q: int, out: int, lse: int, T: int, n_q_heads: int, n_kv_heads: int, head_dim: int, row_ptr: int,
                 nnz: int, block: int, sm_scale: float, workspace: int, ws_bytes: int, stream: int = 0):
    _check("dag_attn_run", lib.dag_attn_run(q, out, lse or None, T, n_q_heads, n_kv_heads, head_dim, row_ptr, nnz, block,
                                            sm_scale, workspace or None, ws_bytes, stream or None))


def kv_causal_attend_workspace_size(pool: int, seq: int, n: int, n_q_heads: int) -> int:
    out = C.c_size_t(0)
    _check("kv_causal_attend_workspace_size",
           lib.kv_causal_attend_workspace_size(pool, seq, n, n_q_heads, C.byref(out)), pool)
    return out.value


def kv_causal_attend(pool: int, seq: int, n: int, n_q_heads: int, q: int, out: int, lse: int, sm_scale: float,
                     workspace: int, ws_bytes: int, stream: int = 0):
    _check("kv_causal_attend", lib.kv_causal_attend(pool, seq, n, n_q_heads, q, out, lse or None, sm_scale,
                                                    workspace or None, ws_bytes, stream or None), pool)


def kv_window_plan(pool: int, seqs, n_q_heads: int, n_steps: int) -> int:
    s = np.ascontiguousarray(np.asarray(seqs, np.int32))
    out = C.c_size_t(0)
    _check("kv_window_plan", lib.kv_window_plan(pool, s.ctypes.data_as(_pi32), len(s), n_q_heads, n_steps,
                                                C.byref(out)), pool)
    return out.value


def kv_window_upload(pool: int, workspace: int, ws_bytes: int, stream: int = 0):
    _check("kv_window_upload", lib.kv_window_upload(pool, workspace or None, ws_bytes, stream or None), pool)


def kv_window_step(pool: int, step: int, k: int, v: int, q: int, out: int, lse: int, sm_scale: float,
                   stream: int = 0):
    _check("kv_window_step", lib.kv_window_step(pool, step, k, v, q, out, lse or None, sm_scale, stream or None),
           pool)


def dag_attn_backward_workspace_size(T: int, n_q_heads: int, n_kv_heads: int, block: int, nnz: int) -> int:
    out = C.c_size_t(0)
    _check("dag_attn_backward_workspace_size",
           lib.dag_attn_backward_workspace_size(T, n_q_heads, n_kv_heads, block, nnz, C.byref(out)))
    return out.value


def dag_attn_backward(q: int, k: int, v: int, out: int, dout: int, lse: int, dq: int, dk: int, dv: int, T: int,
                      n_q_heads: int, n_kv_heads: int, head_dim: int, row_ptr: int, col: int, kind: int, nnz: int,
                      block: int, sm_scale: float, workspace: int, ws_bytes: int, stream: int = 0):
    _check("dag_attn_backward", lib.dag_attn_backward(q, k, v, out, dout, lse, dq, dk, dv, T, n_q_heads, n_kv_heads,
                                                      head_dim, row_ptr, col, kind, nnz, block, sm_scale,
                                                      workspace or None, ws_bytes, stream or None))


# ------------------------------------------------------------------ packed DAG prefill
def select_keep(scores, budget: int, keep=None, workspace=None):
    """keep (uint8 tensor): 1 for the `budget` highest scores, ties to the lower index."""
    import torch
    n = scores.numel()
    if keep is None:
        keep = torch.empty(max(n, 1), dtype=torch.uint8, device=scores.device)[:n]
    if workspace is None:
        workspace = torch.empty(kv_select_workspace_size(n), dtype=torch.uint8, device=scores.device)
    kv_select_keep(scores.data_ptr(), n, budget, keep.data_ptr(), workspace.data_ptr(), workspace.numel(),
                   torch.cuda.current_stream().cuda_stream)
    return keep


class DagMask:
    """Device copy of the CSR block mask of a packed DAG (dag_mask_build on the host)."""

    def __init__(self, segments, edges, T: int, block: int = 64, device: str = "cuda"):
        import torch
        row_ptr, col, kind = dag_mask_build(segments, edges, T, block)
        self.T, self.block, self.nnz = T, block, len(col)
        self.host = (row_ptr, col, kind)
        self.row_ptr = torch.from_numpy(row_ptr).to(device)
        self.col = torch.from_numpy(col if len(col) else np.zeros(1, np.int32)).to(device)
        self.kind = torch.from_numpy(kind if len(kind) else np.zeros(1, np.uint8)).to(device)


def prefill(q, k, v, mask: DagMask, sm_scale: float, out=None, lse=None, workspace=None, with_lse: bool = True):
    """Block-sparse prefill over `mask`.  q [T, Hq, 128], k / v [T, Hkv, 128] bf16 torch
    tensors on the device.  Returns (out [T, Hq, 128] bf16, lse [Hq, T] fp32 or None)."""
    import torch
    T, hq, d = q.shape
    hkv = k.shape[1]
    assert q.is_contiguous() and k.is_contiguous() and v.is_contiguous() and k.shape == v.shape
    assert T == mask.T and q.dtype == torch.bfloat16
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((hq, T), dtype=torch.float32, device=q.device)
    need = dag_attn_workspace_size(T, hq, hkv, mask.block, mask.nnz)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dag_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else 0,
                     T, hq, hkv, d, mask.row_ptr.data_ptr(), mask.col.data_ptr(), mask.kind.data_ptr(), mask.nnz,
                     mask.block, sm_scale, workspace.data_ptr(), workspace.numel(),
                     torch.cuda.current_stream().cuda_stream)
    return out, lse


def prefill_backward(q, k, v, out, dout, lse, mask: DagMask, sm_scale: float, workspace=None):
    """Gradients of `prefill` over `mask`: q / out / dout [T, Hq, 128], k / v [T, Hkv, 128]
    bf16, lse [Hq, T] fp32 from the forward.  Returns (dq [T, Hq, 128], dk, dv [T, Hkv,
    128]) fp32."""
    import torch
    T, hq, d = q.shape
    hkv = k.shape[1]
    for t in (q, k, v, out, dout, lse):
        assert t.is_contiguous()
    assert T == mask.T and q.dtype == torch.bfloat16 and dout.dtype == torch.bfloat16 and lse.dtype == torch.float32
    dq = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((T, hkv, d), dtype=torch.float32, device=q.device)
    dv = torch.empty((T, hkv, d), dtype=torch.float32, device=q.device)
    need = dag_attn_backward_workspace_size(T, hq, hkv, mask.block, mask.nnz)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dag_attn_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), T, hq, hkv, d, mask.row_ptr.data_ptr(),
                      mask.col.data_ptr(), mask.kind.data_ptr(), mask.nnz, mask.block, sm_scale,
                      workspace.data_ptr(), workspace.numel(), torch.cuda.current_stream().cuda_stream)
    return dq, dk, dv


# ------------------------------------------------------------------ torch-backed holder
class Pool:
    """Owns the torch device buffers of one pool (K pages, V pages, workspace) and its handle.

    metadata_only=True creates a host-only pool (no device memory, no device work)."""

    def __init__(self, n_kv_heads: int, head_dim: int, n_pages: int, dtype: str = "bf16", page_size: int = 16,
                 rope_theta: float = 0.0, metadata_only: bool = False, device: str = "cuda"):
        self.dtype = dtype
        self.cfg = make_config(n_kv_heads, head_dim, n_pages, KV_BF16 if dtype == "bf16" else KV_F32, page_size,
                               rope_theta)
        self.k_pages = self.v_pages = self.workspace = None
        self._dec_ws = None
        if metadata_only:
            self.handle = kv_pool_create(self.cfg)
        else:
            import torch
            tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
            nbytes = kv_pool_bytes(self.cfg)
            n_el = nbytes // (2 if dtype == "bf16" else 4)
            self.k_pages = torch.zeros(n_el, dtype=tdt, device=device)
            self.v_pages = torch.zeros(n_el, dtype=tdt, device=device)
            wsb = kv_pool_workspace_size(self.cfg)
            self.workspace = torch.zeros(wsb, dtype=torch.uint8, device=device)
            self.handle = kv_pool_create(self.cfg, self.k_pages.data_ptr(), self.v_pages.data_ptr(),
                                         self.workspace.data_ptr(), wsb)

    def close(self):
        if getattr(self, "handle", None):
            kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _stream() -> int:
        import torch
        return torch.cuda.current_stream().cuda_stream

    def seq_create(self) -> int:
        return kv_seq_create(self.handle)

    def append(self, seq: int, k=None, v=None, positions=None, n: Optional[int] = None):
        if k is None:
            kv_append(self.handle, seq, int(n), 0, 0, positions, 0)
        else:
            assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape
            kv_append(self.handle, seq, k.shape[0], k.data_ptr(), v.data_ptr(), positions, self._stream())

    def append_batch(self, seqs, k=None, v=None):
        """One token onto each listed sequence (row i of k / v for seqs[i])."""
        if k is None:
            kv_append_batch(self.handle, seqs, 0, 0, 0)
        else:
            assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape and k.shape[0] == len(seqs)
            kv_append_batch(self.handle, seqs, k.data_ptr(), v.data_ptr(), self._stream())

    def write(self, seq: int, start: int, k=None, v=None, n: Optional[int] = None):
        if k is None:
            kv_write(self.handle, seq, start, int(n), 0, 0, 0)
        else:
            kv_write(self.handle, seq, start, k.shape[0], k.data_ptr(), v.data_ptr(), self._stream())

    def fork(self, parent: int) -> int:
        return kv_fork(self.handle, parent)

    def mount(self, dst: int, src: int, begin: int, length: int):
        kv_mount(self.handle, dst, src, begin, length)

    def drop(self, seq: int, spans, repos: bool = False) -> np.ndarray:
        st = 0 if self.k_pages is None else self._stream()
        return kv_drop(self.handle, seq, spans, KV_DROP_REPOS if repos else 0, st)

    def drop_batch(self, seqs, spans_per_seq, repos: bool = False):
        st = 0 if self.k_pages is None else self._stream()
        return kv_drop_batch(self.handle, seqs, spans_per_seq, KV_DROP_REPOS if repos else 0, st)

    def score(self, seq: int, q_rep, sm_scale: float, workspace=None):
        """Mean attention of the representative queries q_rep (torch [n_rep, Hq, d] on the
        device) on each own token of `seq`.  Returns a float32 tensor [n_tokens]."""
        import torch
        n_rep, hq, _ = q_rep.shape
        n_tok = self.info(seq)[0]
        need = kv_score_workspace_size(self.handle, seq, n_rep, hq)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q_rep.device)
        scores = torch.empty(max(n_tok, 1), dtype=torch.float32, device=q_rep.device)[:n_tok]
        kv_score(self.handle, seq, q_rep.data_ptr(), n_rep, hq, sm_scale, scores.data_ptr(), workspace.data_ptr(),
                 workspace.numel(), self._stream())
        return scores

    def drop_keep(self, seq: int, keep, repos: bool = False):
        """Drop the tokens whose keep entry (host array, one per own token) is 0."""
        kv_drop_keep(self.handle, seq, keep, KV_DROP_REPOS if repos else 0,
                     0 if self.k_pages is None else self._stream())

    def select_and_drop(self, seq: int, q_rep, sm_scale: float, budget: int, repos: bool = False):
        """Score, keep the `budget` best own tokens, drop the rest.  Returns the keep mask."""
        import torch
        scores = self.score(seq, q_rep, sm_scale)
        keep = select_keep(scores, budget)
        torch.cuda.current_stream().synchronize()
        mask = keep.cpu().numpy()
        self.drop_keep(seq, mask, repos)
        return mask

    def repos(self, seq: int):
        kv_repos(self.handle, seq, 0 if self.k_pages is None else self._stream())

    def rewind(self, seq: int, n: int):
        kv_rewind(self.handle, seq, n)

    def commit(self, seq: int):
        kv_commit(self.handle, seq)

    def release(self, seq: int):
        kv_release(self.handle, seq)

    def info(self, seq: int):
        return kv_seq_info(self.handle, seq)

    def block_table(self, seq: int) -> np.ndarray:
        return kv_block_table(self.handle, seq)

    def positions(self, seq: int) -> np.ndarray:
        return kv_positions(self.handle, seq)

    def refcount(self, page: int) -> int:
        return kv_page_refcount(self.handle, page)

    def free_pages(self) -> int:
        return kv_free_pages(self.handle)

    def read_page(self, page: int, head: int):
        d = self.cfg.head_dim
        dt = np.uint16 if self.dtype == "bf16" else np.float32
        k = np.zeros((16, d), dt)
        v = np.zeros((16, d), dt)
        kv_pool_read_page(self.handle, page, head, k, v, self._stream())
        return k, v

    def sync_status(self) -> int:
        return kv_pool_sync_status(self.handle, self._stream())

    def decode(self, seqs: Sequence[int], q, sm_scale: float, out=None, lse=None, workspace=None):
        """q: torch [n, Hq, d] on the device.  Returns (out, lse)."""
        import torch
        n, hq, d = q.shape
        need = fork_attn_workspace_size(self.handle, seqs, hq)
        if workspace is None:
            if self._dec_ws is None or self._dec_ws.numel() < need:
                self._dec_ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
            workspace = self._dec_ws
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((n, hq), dtype=torch.float32, device=q.device)
        fork_attn_decode(self.handle, seqs, hq, q.data_ptr(), out.data_ptr(), lse.data_ptr(), sm_scale,
                         workspace.data_ptr(), workspace.numel(), self._stream())
        return out, lse

    def causal_attend(self, seq: int, q, sm_scale: float):
        """Attention of the sequence's last q.shape[0] tokens (kv_causal_attend); returns
        (out, lse)."""
        import torch
        n, hq, d = q.shape
        need = kv_causal_attend_workspace_size(self.handle, seq, n, hq)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        out = torch.empty_like(q)
        lse = torch.empty((n, hq), dtype=torch.float32, device=q.device)
        kv_causal_attend(self.handle, seq, n, hq, q.data_ptr(), out.data_ptr(), lse.data_ptr(), sm_scale,
                         ws.data_ptr(), ws.numel(), self._stream())
        return out, lse

    def window(self, seqs: Sequence[int], n_q_heads: int, n_steps: int):
        """Reserve and plan a steady-state decode window (kv_window_plan + kv_window_upload);
        returns the workspace tensor, which must stay alive while the window's steps run."""
        import torch
        need = kv_window_plan(self.handle, seqs, n_q_heads, n_steps)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        kv_window_upload(self.handle, ws.data_ptr(), ws.numel(), self._stream())
        return ws

    def window_step(self, step: int, k, v, q, sm_scale: float, out, lse):
        """One window step: k / v [n, Hkv, d] new rows, q [n, Hq, d]; out / lse written."""
        kv_window_step(self.handle, step, k.data_ptr(), v.data_ptr(), q.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       sm_scale, self._stream())

    def plan_stats(self) -> dict:
        return fork_attn_plan_stats(self.handle)
