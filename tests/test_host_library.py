"""Host logic of libforkattn.so on the CPU (no GPU calls): the C ABI loads and exports
every declared symbol, page-table operations on metadata-only pools are bit-identical
to the oracle's block tables / refcounts / positions / compaction indices, the DAG
block mask equals the oracle's rule-derived block pairs, and the decode planner's
segments and algorithmic byte counts match the workload structure."""
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import fork_attention_decode_amd as fa
import workloads as W
from oracle import pagetable as pt, prefill as pf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "forkattn.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?(?:int|char\s*\*|const char\s*\*)\s*\**\s*([a-z_]+)\s*\(", hdr, re.M))
    names |= set(re.findall(r"^const char\*\s+([a-z_]+)\(", hdr, re.M))
    assert {"kv_pool_create", "fork_attn_decode", "dag_attn_prefill", "kv_last_error"} <= names
    for n in sorted(names):
        assert hasattr(fa.lib, n), n
    assert set(fa.EXPORTED) == names


def _cmp(lib_pool, ora, live):
    assert fa.kv_free_pages(lib_pool) == ora.n_free
    for p in range(ora.capacity):
        assert fa.kv_page_refcount(lib_pool, p) == ora.rc[p], p
    for s in live:
        n, nxt, npg, nm = fa.kv_seq_info(lib_pool, s)
        on, onxt, onp = ora.info(s)
        assert (n, nxt, npg, nm) == (on, onxt, onp, len(ora.seqs[s].mounts))
        assert list(fa.kv_block_table(lib_pool, s)) == ora.block_table(s)
        assert np.array_equal(fa.kv_positions(lib_pool, s), ora.positions(s))


def test_agentrix_example_through_the_library():
    page, src_bytes = 4096, 8 * 2**20
    pool = fa.Pool(1, 2, 2048 * 10, page_size=page, metadata_only=True)
    src = pool.seq_create()
    pool.append(src, n=src_bytes)
    rng = np.random.default_rng(0)
    for _ in range(8):
        c = pool.fork(src)
        pool.write(c, int(rng.integers(0, 2048)) * page + int(rng.integers(0, page - 32)), n=32)
    used = 2048 * 10 - pool.free_pages()
    assert used == 2056 and used * page / 2**20 == 8.03125


OPS = st.lists(st.tuples(st.sampled_from(["append", "fork", "mount", "drop", "repos", "rewind", "release", "write",
                                          "create", "append_pos"]),
                         st.integers(0, 10**6), st.integers(0, 10**6), st.integers(0, 10**6)),
               min_size=1, max_size=40)


def _apply(kind, x, y, z, live, ora):
    """Arguments of one random operation, derived from the (shared) current state."""
    if kind == "create" or not live:
        return (kind,)
    s = live[x % len(live)]
    n_s = ora.seqs[s].n
    if kind == "append":
        return (kind, s, y % 9)
    if kind == "append_pos":
        n = 1 + y % 3
        return (kind, s, n, [z % 50 + 7 * i for i in range(n)])
    if kind == "write":
        return (kind, s, y % (n_s + 2), 1 + z % 4)
    if kind == "mount":
        src = live[y % len(live)]
        return (kind, s, src, z % (ora.seqs[src].n + 2), 1 + (x // 7) % 6)
    if kind in ("drop", "repos"):
        spans = [((z * (j + 3)) % (n_s + 1), 1 + (x + j) % 5) for j in range(y % 3)] if kind == "drop" else []
        return ("drop", s, spans, kind == "repos" or z % 2 == 1)
    if kind == "rewind":
        return (kind, s, y % (n_s + 2))
    return (kind, s)


def _run_oracle(op, ora):
    k = op[0]
    if k == "create": return ora.create()
    if len(op) == 1: return None
    if k == "append": return ora.append(op[1], op[2])
    if k == "append_pos": return ora.append(op[1], op[2], pos=op[3])
    if k == "fork": return ora.fork(op[1])
    if k == "write": return ora.write(op[1], op[2], op[3])
    if k == "mount": return ora.mount(*op[1:])
    if k == "drop": return ora.drop(op[1], op[2], repos=op[3])
    if k == "rewind": return ora.rewind(op[1], op[2])
    if k == "release": return ora.release(op[1])


def _run_lib(op, pool):
    k = op[0]
    if k == "create": return fa.kv_seq_create(pool)
    if len(op) == 1: return None
    if k == "append": return fa.kv_append(pool, op[1], op[2])
    if k == "append_pos": return fa.kv_append(pool, op[1], op[2], positions=op[3])
    if k == "fork": return fa.kv_fork(pool, op[1])
    if k == "write": return fa.kv_write(pool, op[1], op[2], op[3])
    if k == "mount": return fa.kv_mount(pool, *op[1:])
    if k == "drop": return fa.kv_drop(pool, op[1], op[2], fa.KV_DROP_REPOS if op[3] else 0)
    if k == "rewind": return fa.kv_rewind(pool, op[1], op[2])
    if k == "release": return fa.kv_release(pool, op[1])


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(ops=OPS, page=st.integers(1, 5), cap=st.integers(1, 24))
def test_random_ops_bit_exact_against_oracle(ops, page, cap):
    ora = pt.PageTable(cap, page)
    pool = fa.kv_pool_create(fa.make_config(1, 2, cap, page_size=page))
    try:
        ora.create(); fa.kv_seq_create(pool)
        for kind, x, y, z in ops:
            live = [i for i, s in enumerate(ora.seqs) if s.live]
            op = _apply(kind, x, y, z, live, ora)
            err_o = err_l = None
            r_o = r_l = None
            try:
                r_o = _run_oracle(op, ora)
            except pt.OOM:
                err_o = fa.KV_ERR_OOM
            except pt.Invalid:
                err_o = fa.KV_ERR_INVALID
            try:
                r_l = _run_lib(op, pool)
            except fa.ForkAttnError as e:
                err_l = e.status
            assert err_o == err_l, (op, err_o, err_l)
            if op[0] in ("create", "fork") and err_o is None:
                assert r_o == r_l                      # handles assigned in creation order
            if op[0] == "drop" and err_o is None:
                assert np.array_equal(r_o, r_l)         # compaction indices
            _cmp(pool, ora, [i for i, s in enumerate(ora.seqs) if s.live])
    finally:
        fa.kv_pool_destroy(pool)


@pytest.mark.parametrize("make", [
    lambda: W.shared_prefix_fork(),
    lambda: W.octopus_dag(),
    lambda: W.drop_scenario(requests=3, ctx=20000, span_min=300, span_max=1200, seed=4),
])
def test_workload_scenarios_bit_exact(make, monkeypatch):
    import workloads
    # metadata only: avoid drawing the token values
    sc = make()
    ora, drops = pt.replay(sc, with_data=False)
    pool = fa.Pool(sc.n_kv_heads, sc.head_dim, sc.n_pages, page_size=sc.page_size, rope_theta=sc.rope_theta,
                   metadata_only=True)
    kept = []
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "append":
            blk = sc.blocks[op[2]]
            pool.append(op[1], n=len(blk.pos), positions=blk.pos)
        elif op[0] == "fork":
            pool.fork(op[1])
        elif op[0] == "mount":
            pool.mount(*op[1:])
        elif op[0] == "drop":
            kept.append(pool.drop(op[1], op[2], repos=op[3]))
    for a, b in zip(drops, kept):
        assert np.array_equal(a, b)
    _cmp(pool.handle, ora, [i for i, s in enumerate(ora.seqs) if s.live])


def test_planner_segments_and_bytes_shared_prefix():
    sc = W.fork_scenario(prefix=32768, branches=16, private=2048)
    pool = fa.Pool(8, 128, sc.n_pages, rope_theta=1e6, metadata_only=True)
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "append":
            pool.append(op[1], n=len(sc.blocks[op[2]].pos))
        elif op[0] == "fork":
            pool.fork(op[1])
    fa.fork_attn_workspace_size(pool.handle, sc.queries, 32)
    st_ = pool.plan_stats()
    assert st_["segments"] == 17                      # one public + 16 private
    assert st_["unique_kv_bytes"] == 268435456        # each shared page counted once
    assert st_["rows"] == 16 * 32


def test_planner_octopus_dag_bytes():
    sc = W.dag_scenario()
    pool = fa.Pool(8, 128, sc.n_pages, rope_theta=1e6, metadata_only=True)
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "append":
            pool.append(op[1], n=len(sc.blocks[op[2]].pos))
        elif op[0] == "fork":
            pool.fork(op[1])
        elif op[0] == "mount":
            pool.mount(*op[1:])
    fa.fork_attn_workspace_size(pool.handle, sc.queries, 32)
    st_ = pool.plan_stats()
    assert st_["unique_kv_bytes"] == 536870912
    # root + per thread (own first half) + per thread (terminal block with its mounters)
    assert st_["segments"] == 1 + 8 + 8


@pytest.mark.parametrize("args", [
    dict(prefix=256, branches=4, branch_len=128, n_edges=3, edge_len=64, block=32),
    dict(prefix=128, branches=3, branch_len=[64, 96, 70], n_edges=2, edge_len=32, block=32),
    dict(prefix=64, branches=1, branch_len=64, n_edges=0, edge_len=32, block=16),
])
def test_dag_mask_matches_oracle_blocks(args):
    p = W.prefill_inputs(with_data=False, **args)
    blk = args["block"]
    row_ptr, col, kind = fa.dag_mask_build(p.segments, p.edges, p.T, blk)
    need = pf.block_pairs(p.segments, p.edges, p.T, blk)
    nb = need.shape[0]
    got = np.zeros_like(need)
    for qb in range(nb):
        cols = col[row_ptr[qb]:row_ptr[qb + 1]]
        assert np.all(np.diff(cols) > 0)
        got[qb, cols] = True
        assert kind[row_ptr[qb + 1] - 1] == 1 and cols[-1] == qb and np.all(kind[row_ptr[qb]:row_ptr[qb + 1] - 1] == 0)
    assert np.array_equal(got, need)
    # token level: FULL blocks fully visible, DIAG blocks exactly causal
    mask = pf.visible_mask(p.segments, p.edges, p.T)
    for qb in range(nb):
        for j in range(row_ptr[qb], row_ptr[qb + 1]):
            kb = col[j]
            sub = mask[qb * blk:(qb + 1) * blk, kb * blk:(kb + 1) * blk]
            if kind[j] == 0:
                assert sub.all()
            else:
                assert np.array_equal(sub, np.tril(np.ones_like(sub)))


def test_dag_mask_full_workload_counts():
    p = W.dag_prefill(with_data=False)
    row_ptr, col, kind = fa.dag_mask_build(p.segments, p.edges, p.T, 64)
    assert len(col) == 410240 and int(kind.sum()) == 1280 and len(row_ptr) == 1281


def test_error_paths_leave_state():
    pool = fa.Pool(1, 2, 4, page_size=4, metadata_only=True)
    a = pool.seq_create()
    pool.append(a, n=10)
    with pytest.raises(fa.ForkAttnError) as e:
        pool.append(a, n=20)
    assert e.value.status == fa.KV_ERR_OOM
    assert pool.info(a) == (10, 10, 3, 0) and pool.free_pages() == 1
    with pytest.raises(fa.ForkAttnError) as e:
        pool.fork(99)
    assert e.value.status == fa.KV_ERR_NOT_FOUND
    with pytest.raises(fa.ForkAttnError) as e:
        pool.drop(a, [(5, 10)])
    assert e.value.status == fa.KV_ERR_INVALID
    pool.release(a)
    with pytest.raises(fa.ForkAttnError) as e:
        pool.release(a)
    assert e.value.status == fa.KV_ERR_NOT_FOUND
    assert pool.free_pages() == 4
    with pytest.raises(fa.ForkAttnError) as e:
        fa.fork_attn_decode(pool.handle, [0], 1, 1, 1, 0, 1.0, 1, 1)
    assert e.value.status in (fa.KV_ERR_INVALID, fa.KV_ERR_NOT_FOUND)


@pytest.mark.parametrize("make,n_steps", [
    (lambda: W.fork_scenario(prefix=517, branches=5, private=[0, 3, 16, 30, 1], hq=8, hkv=2, d=128, seed=71), 20),
    (lambda: W.dag_scenario(root=300, threads=3, private=90, mounts_per_thread=2, mount_len=33, hq=8, hkv=2, d=128,
                            seed=72), 37),
])
def test_window_reservation_equals_rounds_of_appends(make, n_steps):
    # kv_window_plan changes the page table exactly as n_steps rounds of one append per
    # sequence (in list order): shared partial tails copied first, pages lowest-first
    sc = make()
    sc.n_pages += 64
    ora, _ = pt.replay(sc, with_data=False)
    pool = fa.Pool(sc.n_kv_heads, sc.head_dim, sc.n_pages, page_size=sc.page_size, rope_theta=sc.rope_theta,
                   metadata_only=True)
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "append":
            blk = sc.blocks[op[2]]
            pool.append(op[1], n=len(blk.pos), positions=blk.pos)
        elif op[0] == "fork":
            pool.fork(op[1])
        elif op[0] == "mount":
            pool.mount(*op[1:])
    live = [i for i, s in enumerate(ora.seqs) if s.live]
    seqs = [i for i in live if i != 0][::-1]  # not in creation order
    need = fa.kv_window_plan(pool.handle, seqs, sc.n_q_heads, n_steps)
    assert need > 0
    for _ in range(n_steps):
        for b in seqs:
            ora.append(b, 1)
    _cmp(pool.handle, ora, live)


@pytest.mark.parametrize("make", [
    lambda: W.fork_scenario(prefix=517, branches=5, private=[0, 3, 16, 30, 1], hq=8, hkv=2, d=128, seed=73),
    lambda: W.dag_scenario(root=300, threads=3, private=90, mounts_per_thread=2, mount_len=33, hq=8, hkv=2, d=128,
                           seed=74),
])
def test_append_batch_equals_single_appends_in_list_order(make):
    # kv_append_batch = one single-token append per listed sequence, in list order: forks
    # sharing a partial tail (the first copies it, the next then owns it alone), full tails
    # taking new pages, an empty root, repeated steps crossing page boundaries
    sc = make()
    sc.n_pages += 96
    ora, _ = pt.replay(sc, with_data=False)
    pool = fa.Pool(sc.n_kv_heads, sc.head_dim, sc.n_pages, page_size=sc.page_size, rope_theta=sc.rope_theta,
                   metadata_only=True)
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "append":
            blk = sc.blocks[op[2]]
            pool.append(op[1], n=len(blk.pos), positions=blk.pos)
        elif op[0] == "fork":
            pool.fork(op[1])
        elif op[0] == "mount":
            pool.mount(*op[1:])
    assert pool.seq_create() == ora.create()  # an empty root
    live = [i for i, s in enumerate(ora.seqs) if s.live]
    seqs = live[::-1]
    for _ in range(19):
        pool.append_batch(seqs)
        for b in seqs:
            ora.append(b, 1)
        _cmp(pool.handle, ora, live)


def test_append_batch_rejections_leave_state():
    pool = fa.Pool(1, 2, 6, page_size=4, metadata_only=True)
    a = pool.seq_create()
    pool.append(a, n=5)
    b = pool.fork(a)
    c = pool.fork(a)
    pool.append(a, n=3)  # 4-token pages: a copies the shared tail (3 pages in use)
    state = lambda: ([list(fa.kv_block_table(pool.handle, s)) for s in (a, b, c)], pool.free_pages())
    before = state()
    for bad, status in (([b, b], fa.KV_ERR_INVALID), ([b, 99], fa.KV_ERR_NOT_FOUND), (list(range(7)), fa.KV_ERR_INVALID)):
        with pytest.raises(fa.ForkAttnError) as e:
            fa.kv_append_batch(pool.handle, bad)
        assert e.value.status == status, bad
        assert state() == before
    pool.append(c, n=3)  # c copies the shared tail too, b then owns the original alone
    pool.append(b, n=4)  # b fills it in place and takes a new page: one page left
    before = state()  # a and c are at page boundaries: the batch needs two new pages
    with pytest.raises(fa.ForkAttnError) as e:
        fa.kv_append_batch(pool.handle, [a, b, c])
    assert e.value.status == fa.KV_ERR_OOM
    assert state() == before


def test_window_oom_and_duplicates_leave_state():
    pool = fa.Pool(1, 2, 6, page_size=4, metadata_only=True)
    a = pool.seq_create()
    pool.append(a, n=5)
    b = pool.fork(a)
    before = [list(fa.kv_block_table(pool.handle, s)) for s in (a, b)]
    with pytest.raises(fa.ForkAttnError) as e:
        fa.kv_window_plan(pool.handle, [a, b], 2, 8)  # 2 tail copies + 2 x 2 new pages > 4 free
    assert e.value.status == fa.KV_ERR_OOM
    with pytest.raises(fa.ForkAttnError) as e:
        fa.kv_window_plan(pool.handle, [a, a], 2, 1)
    assert e.value.status == fa.KV_ERR_INVALID
    assert [list(fa.kv_block_table(pool.handle, s)) for s in (a, b)] == before


def test_new_entry_points_reject_bad_arguments():
    # window, causal attention and the prefill backward fail with a status, before any
    # device work, on metadata-only pools and bad shapes
    pool = fa.Pool(1, 2, 8, page_size=4, metadata_only=True)
    a = pool.seq_create()
    pool.append(a, n=6)
    with pytest.raises(fa.ForkAttnError) as e:
        fa.kv_window_upload(pool.handle, 1, 1 << 20)  # nothing planned
    assert e.value.status == fa.KV_ERR_INVALID
    with pytest.raises(fa.ForkAttnError) as e:
        fa.kv_window_step(pool.handle, 0, 1, 1, 1, 1, 0, 1.0)
    assert e.value.status == fa.KV_ERR_INVALID
    with pytest.raises(fa.ForkAttnError) as e:
        fa.kv_causal_attend_workspace_size(pool.handle, a, 7, 2)  # more tokens than the sequence holds
    assert e.value.status == fa.KV_ERR_INVALID
    assert fa.kv_causal_attend_workspace_size(pool.handle, a, 6, 2) > 0  # metadata pools can plan
    with pytest.raises(fa.ForkAttnError) as e:
        fa.kv_causal_attend(pool.handle, a, 6, 2, 1, 1, 0, 1.0, 1, 1 << 20)
    assert e.value.status == fa.KV_ERR_INVALID  # no KV data
    with pytest.raises(fa.ForkAttnError) as e:
        fa.dag_attn_backward_workspace_size(64, 3, 2, 64, 1)  # Hq not a multiple of Hkv
    assert e.value.status == fa.KV_ERR_INVALID
    with pytest.raises(fa.ForkAttnError) as e:
        fa.dag_attn_backward(1, 1, 1, 1, 1, 1, 1, 1, 1, 64, 4, 2, 64, 1, 1, 1, 1, 64, 1.0, 1, 1 << 30)
    assert e.value.status == fa.KV_ERR_UNSUPPORTED  # head_dim 64
    with pytest.raises(fa.ForkAttnError) as e:
        fa.dag_attn_backward(1, 1, 1, 1, 1, 1, 1, 1, 1, 64, 4, 2, 128, 1, 1, 1, 1, 64, 0.0, 1, 1 << 30)
    assert e.value.status == fa.KV_ERR_INVALID  # scale
    with pytest.raises(fa.ForkAttnError) as e:
        fa.dag_attn_backward(1, 1, 1, 1, 1, 1, 1, 1, 1, 64, 4, 2, 128, 1, 1, 1, 1, 64, 1.0, 1, 16)
    assert e.value.status == fa.KV_ERR_WORKSPACE
    fa.dag_attn_backward(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 4, 2, 128, 0, 0, 0, 0, 64, 1.0, 0, 0)  # T = 0: nothing to do
    assert pool.info(a)[0] == 6


def test_bench_refuses_more_than_one_gpu():
    # the bench measures one GPU; a request for several exits with a message, before any
    # GPU work
    import subprocess
    import sys
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def test_append_batch_copy_source_written_in_place_by_a_later_sequence():
    # a has 40 tokens (pages of 16), b = fork(a) rewound to 36: page 2 is shared, a's
    # token 36 sits in its slot 4.  append_batch([a, b]): a copies page 2 (its token goes
    # to slot 8 of the copy), after which b owns page 2 alone and writes slot 4 in place.
    # The same decisions as two single appends in list order.
    pool = fa.Pool(1, 2, 16, metadata_only=True)
    ora = pt.PageTable(16, 16)
    a = pool.seq_create()
    assert ora.create() == a
    pool.append(a, n=40)
    ora.append(a, 40)
    b = pool.fork(a)
    assert ora.fork(a) == b
    pool.rewind(b, 36)
    ora.rewind(b, 36)
    shared = list(fa.kv_block_table(pool.handle, a))[2]
    assert fa.kv_page_refcount(pool.handle, shared) == 2
    pool.append_batch([a, b])
    ora.append(a, 1)
    ora.append(b, 1)
    _cmp(pool.handle, ora, [a, b])
    ta, tb = list(fa.kv_block_table(pool.handle, a)), list(fa.kv_block_table(pool.handle, b))
    assert ta[:2] == tb[:2] and ta[2] != shared and tb[2] == shared  # a copied, b wrote in place
    assert fa.kv_page_refcount(pool.handle, shared) == 1


@pytest.mark.parametrize("make", [
    lambda: W.drop_scenario(requests=4, ctx=700, frac=0.4, span_min=17, span_max=120, hq=4, hkv=2, d=128, seed=91,
                            repos=True),
    lambda: W.fork_scenario(prefix=517, branches=4, private=[60, 200, 9, 0], hq=8, hkv=2, d=128, seed=92),
    lambda: W.dag_scenario(root=300, threads=4, private=200, mounts_per_thread=2, mount_len=70, hq=8, hkv=2, d=128,
                           seed=93),
])
@pytest.mark.parametrize("repos", [True, False])
def test_drop_batch_equals_single_drops_in_list_order(make, repos):
    # kv_drop_batch = one kv_drop per listed sequence, in list order: independent requests,
    # forks sharing a prefix (a later drop may rewrite in place a page an earlier one
    # released), mounted threads (copies); compaction indices, tables, refcounts, positions
    sc = make()
    sc.ops = [op for op in sc.ops if op[0] != "drop"]
    sc.n_pages += 200
    ora, _ = pt.replay(sc, with_data=False)
    pool = fa.Pool(sc.n_kv_heads, sc.head_dim, sc.n_pages, page_size=sc.page_size, rope_theta=sc.rope_theta,
                   metadata_only=True)
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "append":
            blk = sc.blocks[op[2]]
            pool.append(op[1], n=len(blk.pos), positions=blk.pos)
        elif op[0] == "fork":
            pool.fork(op[1])
        elif op[0] == "mount":
            pool.mount(*op[1:])
    live = [i for i, s in enumerate(ora.seqs) if s.live]
    rng = np.random.default_rng(94)
    seqs = list(rng.permutation(live))
    spans = []
    for s in seqs:
        n = ora.seqs[s].n
        sp = [(int(b), int(min(n - b, rng.integers(1, 40)))) for b in sorted(rng.integers(0, max(1, n), 3))] if n else []
        spans.append(sp)
    kept = pool.drop_batch(seqs, spans, repos=repos)
    for s, sp, k in zip(seqs, spans, kept):
        assert np.array_equal(k, ora.drop(s, sp, repos=repos)), s
    _cmp(pool.handle, ora, live)


def test_drop_batch_rejections_leave_state():
    pool = fa.Pool(1, 2, 8, page_size=4, metadata_only=True)
    a = pool.seq_create()
    pool.append(a, n=9)
    b = pool.fork(a)
    c = pool.seq_create()
    pool.append(c, n=6)
    state = lambda: ([list(fa.kv_block_table(pool.handle, s)) for s in (a, b, c)], pool.free_pages(),
                     [list(fa.kv_positions(pool.handle, s)) for s in (a, b, c)])
    before = state()
    for seqs, spans, status in (([a, a], [[(0, 1)], [(1, 1)]], fa.KV_ERR_INVALID),
                                ([a, 9], [[(0, 1)], []], fa.KV_ERR_NOT_FOUND),
                                ([c, a], [[(0, 1)], [(5, 9)]], fa.KV_ERR_INVALID),  # the second span is bad
                                ([a, b], [[(0, 1)], [(0, 1)]], fa.KV_ERR_OOM)):    # copies of both exceed 1 free page
        with pytest.raises(fa.ForkAttnError) as e:
            pool.drop_batch(seqs, spans, repos=True)
        assert e.value.status == status, (seqs, spans)
        assert state() == before


def test_patched_plan_totals_equal_a_fresh_plan():
    # appends into pages a branch owns alone patch the cached decode plan; its totals
    # (unique KV bytes, rows, segments, chunks) equal those of a plan built from scratch,
    # and any other change (a drop) makes the next call replan
    sc = W.fork_scenario(prefix=517, branches=4, private=[0, 3, 16, 29], hq=8, hkv=2, d=128, seed=41)
    sc.n_pages += 80
    pool = fa.Pool(sc.n_kv_heads, sc.head_dim, sc.n_pages, metadata_only=True)
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "append":
            pool.append(op[1], n=len(sc.blocks[op[2]].pos), positions=sc.blocks[op[2]].pos)
        elif op[0] == "fork":
            pool.fork(op[1])
    seqs = list(sc.queries)
    for step in range(45):
        fa.fork_attn_workspace_size(pool.handle, seqs, 8)
        pool.append_batch(seqs)
    fa.fork_attn_workspace_size(pool.handle, seqs, 8)
    patched = pool.plan_stats()
    assert patched["patched_changes"] >= 40
    fa.fork_attn_workspace_size(pool.handle, seqs[::-1], 8)  # another query list: a fresh plan
    fa.fork_attn_workspace_size(pool.handle, seqs, 8)
    fresh = pool.plan_stats()
    assert fresh["patched_changes"] == 0
    for key in ("unique_kv_bytes", "rows", "segments", "chunks"):
        assert patched[key] == fresh[key], key
    pool.drop(seqs[0], [(0, 3)])
    fa.fork_attn_workspace_size(pool.handle, seqs, 8)
    assert pool.plan_stats()["patched_changes"] == 0
