"""GPU parity of fork_attn_decode (HIP path through the C ABI) against the fp64 oracle.

Bars: every output element and LSE within the decode error model's bars
(tests/harness.py: decode_bars, derived from the kernel's arithmetic: bf16 P, fp32
sums), and within the coarse gate (bf16 max-abs 2e-2 / mean-abs 2e-3, fp32 pools
max-abs 1e-4, LSE 2e-3).  Planted-key cases (one key singled out per row, so the row's
output is that key's value: a closed form) cover every chunk slot of the longest work
items, at small size with a one-compute-unit plan and at full size.  Integer state
(block tables, refcounts) bit-exact.  Every case prints its name first.
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import (build_device_pool, check_close, check_decode_both, check_decode_model, oracle_decode,
                           out_to_f64, plant_queries, subscenario, to_torch)

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX, LSE_MAX = 2e-2, 2e-3, 1e-4, 2e-3


def _run(sc, label, q=None, n_cu=None):
    import torch
    import fork_attention_decode_amd as fa
    print(f"[case] {label}: {sc.name} Hq={sc.n_q_heads} Hkv={sc.n_kv_heads} d={sc.head_dim} {sc.dtype}", flush=True)
    pool, _ = build_device_pool(sc)
    if n_cu is not None:
        fa.kv_pool_set_compute_units(pool.handle, n_cu)
    out, lse = pool.decode(sc.queries, to_torch(sc.q if q is None else q, sc.dtype), sc.sm_scale)
    torch.cuda.synchronize()
    return pool, out_to_f64(out, sc.dtype), lse.double().cpu().numpy()


def _check(sc, o, lse, label, rows=None, q=None):
    ro, rl, a, s_abs = oracle_decode(sc, rows, with_magnitudes=True, q=q)
    if rows is not None:
        o, lse = o[rows], lse[rows]
    if sc.dtype == "bf16":
        mx, mn = check_close(o, ro, BF16_MAX, BF16_MEAN, label)
    else:
        mx, mn = check_close(o, ro, F32_MAX, F32_MAX, label)
    check_close(lse, rl, LSE_MAX, LSE_MAX, label + " lse")
    wo, wl = check_decode_model(o, lse, ro, rl, a, s_abs, sc.head_dim, sc.dtype, label)
    print(f"[ok] {label}: max-abs {mx:.3g} mean-abs {mn:.3g}; error / model bar: O {wo:.3f}, LSE {wl:.3f}",
          flush=True)


def _check_planted(sc, o, vp, label):
    """Closed form: a planted row's output is the planted key's value (bf16 values are
    exact in the output type; the other keys carry ~e^-20 of the weight)."""
    err = np.abs(o - vp)
    bad = err > 2.0 ** -8 * np.abs(vp) + 1e-6
    assert not bad.any(), f"{label}: {int(bad.sum())} planted elements differ from v_j, rows {np.argwhere(bad)[:4, :2].tolist()}"


def test_tiny_fork_fp32():
    sc = W.tiny_fork()
    pool, o, lse = _run(sc, "tiny fork fp32")
    _check(sc, o, lse, "tiny fork fp32")
    st = pool.plan_stats()
    assert st["unique_kv_bytes"] == 262144 and st["segments"] == 5


@pytest.mark.parametrize("private", [[33, 0, 17, 64, 1, 300], [16, 16, 16], [1]])
def test_ragged_fork_bf16(private):
    sc = W.fork_scenario(prefix=517, branches=len(private), private=private, hq=8, hkv=2, d=128, seed=3)
    pool, o, lse = _run(sc, f"ragged fork {private}")
    _check(sc, o, lse, f"ragged fork {private}")


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4, 5])
def test_random_trees_bf16(seed):
    # seeded random shapes: forks over a shared prefix (odd seeds: a DAG of threads with
    # mounts), head counts, and for some seeds a plan for 1 or 3 compute units (long work
    # items, so chunk slots past 64 are used)
    rng = np.random.default_rng(2000 + seed)
    hq, hkv = [(8, 2), (4, 1), (16, 4), (8, 8), (12, 2), (32, 8)][seed]
    if seed % 2 == 0:
        branches = int(rng.integers(1, 7))
        private = [int(x) for x in rng.integers(0, 400, size=branches)]
        sc = W.fork_scenario(prefix=int(rng.integers(1, 3000)), branches=branches, private=private, hq=hq, hkv=hkv,
                             d=128, seed=20 + seed)
    else:
        threads = int(rng.integers(2, 6))
        mpt = int(rng.integers(1, threads))
        private = int(rng.integers(40, 400))
        sc = W.dag_scenario(root=int(rng.integers(1, 2000)), threads=threads, private=private, mounts_per_thread=mpt,
                            mount_len=int(rng.integers(1, private + 1)), hq=hq, hkv=hkv, d=128, seed=20 + seed)
    n_cu = [None, 3, None, 1, None, None][seed]
    label = f"random tree seed={seed} Hq={hq} Hkv={hkv} n_cu={n_cu}"
    pool, o, lse = _run(sc, label, n_cu=n_cu)
    _check(sc, o, lse, label)


def test_edge_shapes_bf16():
    """Degenerate and maximal shapes: 64 query heads on one KV head (a work item's full 64
    rows from one reader), a branch with no private token, the root decoding beside its
    forks, one sequence listed twice, and an empty query list."""
    import dataclasses
    import torch
    sc = W.fork_scenario(prefix=100, branches=3, private=[0, 5, 40], hq=64, hkv=1, d=128, seed=11)
    pool, o, lse = _run(sc, "64 query heads on one KV head")
    _check(sc, o, lse, "64 query heads on one KV head")
    # root (0), branch 2 twice, branch 1: rows 1 and 2 read the same context with different queries
    sc2 = dataclasses.replace(sc, queries=[0, 2, 2, 1], q=sc.q[[0, 1, 2, 0]])
    out, lse2 = pool.decode(sc2.queries, to_torch(sc2.q, sc2.dtype), sc2.sm_scale)
    torch.cuda.synchronize()
    _check(sc2, out_to_f64(out, sc2.dtype), lse2.double().cpu().numpy(), "root + repeated sequence")
    # an empty query list: no launch, nothing written
    q0 = torch.empty((0, sc.n_q_heads, sc.head_dim), dtype=torch.bfloat16, device="cuda")
    out0, lse0 = pool.decode([], q0, sc.sm_scale)
    torch.cuda.synchronize()
    assert out0.shape == (0, sc.n_q_heads, sc.head_dim) and lse0.shape == (0, sc.n_q_heads)


def test_many_rows_split_groups_bf16():
    # 20 branches x G=8 rows -> 160 rows on the shared prefix: three reader groups
    sc = W.fork_scenario(prefix=300, branches=20, private=5, hq=16, hkv=2, d=128, seed=9)
    pool, o, lse = _run(sc, "20 branches G=8")
    _check(sc, o, lse, "20 branches G=8")


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f32")])
def test_other_head_dims(d, dtype):
    sc = W.fork_scenario(prefix=200, branches=3, private=[7, 40, 0], hq=4, hkv=2, d=d, dtype=dtype,
                         rope_theta=1e4, seed=5)
    pool, o, lse = _run(sc, f"d={d} {dtype}")
    _check(sc, o, lse, f"d={d} {dtype}")


def test_dag_with_mounts_bf16():
    sc = W.dag_scenario(root=700, threads=5, private=333, mounts_per_thread=3, mount_len=131, hq=8, hkv=2, d=128,
                        seed=11)
    pool, o, lse = _run(sc, "small DAG with mounts")
    _check(sc, o, lse, "small DAG with mounts")


def test_append_pages_and_cow_contents():
    import torch
    sc = W.fork_scenario(prefix=37, branches=2, private=[5, 20], hq=4, hkv=2, d=128, seed=2)
    print("[case] page contents after append / copy-on-write", flush=True)
    pool, _ = build_device_pool(sc)
    from oracle import pagetable as pt
    ora, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, "bf16"))
    for s in range(3):
        assert list(pool.block_table(s)) == ora.block_table(s)
        for L, page in enumerate(ora.block_table(s)):
            n_valid = min(16, ora.seqs[s].n - 16 * L)
            for h in range(2):
                k, v = pool.read_page(page, h)
                assert np.array_equal(W.bf16_bits_to_f64(k[:n_valid]), ora.kdata[page][:n_valid, h])
                assert np.array_equal(W.bf16_bits_to_f64(v[:n_valid]), ora.vdata[page][:n_valid, h])


def test_plan_cache_reuse_and_second_call():
    import torch
    sc = W.fork_scenario(prefix=100, branches=3, private=9, hq=8, hkv=2, d=128, seed=4)
    print("[case] repeated decode calls reuse the cached plan", flush=True)
    pool, _ = build_device_pool(sc)
    q = to_torch(sc.q, "bf16")
    o1, l1 = pool.decode(sc.queries, q, sc.sm_scale)
    o2, l2 = pool.decode(sc.queries, q, sc.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_partials_merge_equals_decode():
    import torch
    import fork_attention_decode_amd as fa
    sc = W.dag_scenario(root=300, threads=3, private=90, mounts_per_thread=2, mount_len=33, hq=8, hkv=2, d=128,
                        seed=6)
    print("[case] fork_attn_partials + fork_attn_merge == fork_attn_decode", flush=True)
    pool, _ = build_device_pool(sc)
    q = to_torch(sc.q, "bf16")
    o1, l1 = pool.decode(sc.queries, q, sc.sm_scale)
    ws = pool._dec_ws
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    st = torch.cuda.current_stream().cuda_stream
    fa.fork_attn_partials(pool.handle, sc.queries, 8, q.data_ptr(), sc.sm_scale, ws.data_ptr(), ws.numel(), st)
    fa.fork_attn_merge(pool.handle, sc.queries, 8, o2.data_ptr(), l2.data_ptr(), ws.data_ptr(), ws.numel(), st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_shared_prefix_full_size():
    sc = W.shared_prefix_fork()
    pool, o, lse = _run(sc, "shared-prefix fork decode, full size")
    st = pool.plan_stats()
    assert st["unique_kv_bytes"] == 268435456
    _check(sc, o, lse, "shared-prefix fork decode, full size")


def test_octopus_dag_full_size():
    sc = W.octopus_dag()
    pool, o, lse = _run(sc, "Octopus DAG decode, full size")
    st = pool.plan_stats()
    assert st["unique_kv_bytes"] == 536870912 and st["longest_item_chunks"] == 128
    _check(sc, o, lse, "Octopus DAG decode, full size")


def test_long_items_planted_keys_small():
    # a one-compute-unit plan cuts the 128-page shared prefix into one 128-chunk item per
    # KV head, so chunk slots 64..127 (the second chunk-metadata register) are read at
    # small size; every row singles out a key in a different chunk slot, half of them in
    # slots 64..127, the rest in the low slots and the private tails
    sc = W.fork_scenario(prefix=2048, branches=3, private=[40, 0, 300], hq=8, hkv=2, d=128, seed=12)
    n, hq = len(sc.queries), sc.n_q_heads
    ctx = [2048 + 40, 2048, 2048 + 300]
    idx = [[16 * (64 + 5 * (4 * i + h // 2)) + h if h % 2 == 0 else (16 * (21 * i + 3 * h) + 5) % ctx[i]
            for h in range(hq)] for i in range(n)]
    idx[1][6] = 16 * 127 + 15  # the last slot of the last chunk
    idx[0][7], idx[2][5] = 2048 + 39, 2048 + 299  # the private tails' last tokens
    qs, vp, idx = plant_queries(sc, None, idx=idx)
    pool, o, lse = _run(sc, "planted keys over 128-chunk items", q=qs, n_cu=1)
    assert pool.plan_stats()["longest_item_chunks"] == 128
    _check_planted(sc, o, vp, "planted keys over 128-chunk items")
    _check(sc, o, lse, "planted keys over 128-chunk items", q=qs)


@pytest.mark.parametrize("make", [W.shared_prefix_fork, W.octopus_dag], ids=["shared_prefix", "octopus_dag"])
def test_planted_keys_full_size(make):
    # every row (branch, query head) of the full-size workload singles out one key drawn
    # uniformly from its context: a page missing from a work item, read twice, or read
    # from the wrong place moves that row's output by O(1)
    sc = make()
    qs, vp, idx = plant_queries(sc, np.random.default_rng(99))
    pool, o, lse = _run(sc, f"planted keys, {sc.name}, full size", q=qs)
    _check_planted(sc, o, vp, f"planted keys, {sc.name}")
    _check(sc, o, lse, f"planted keys, {sc.name}", q=qs)


def test_append_batch_contents_and_decode():
    # kv_append_batch, a few steps of one token per branch (a shared partial tail copied
    # by the first fork, then owned by the second; page boundaries crossed): every page's
    # K / V against the oracle's pages after the same single appends, and a decode after
    import torch
    from oracle import attention as att, pagetable as pt
    sc = W.fork_scenario(prefix=37, branches=3, private=[0, 0, 14], hq=8, hkv=2, d=128, seed=5)
    sc.n_pages += 16
    print("[case] kv_append_batch: contents and a decode", flush=True)
    pool, _ = build_device_pool(sc)
    ora, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, "bf16"))
    seqs = [2, 1, 3, 0]
    rng = np.random.default_rng(6)
    f = W.bf16_bits_to_f64
    for _ in range(5):
        kb = W.to_bf16_bits(rng.standard_normal((len(seqs), 2, 128)) / np.sqrt(128))
        vb = W.to_bf16_bits(rng.standard_normal((len(seqs), 2, 128)))
        pool.append_batch(seqs, to_torch(kb, "bf16"), to_torch(vb, "bf16"))
        for i, b in enumerate(seqs):
            ora.append(b, 1, k=f(kb[i:i + 1]), v=f(vb[i:i + 1]))
    torch.cuda.synchronize()
    for s in seqs:
        assert list(pool.block_table(s)) == ora.block_table(s), s
        for L, page in enumerate(ora.block_table(s)):
            n_valid = min(16, ora.seqs[s].n - 16 * L)
            for h in range(2):
                k, v = pool.read_page(page, h)
                assert np.array_equal(f(k[:n_valid]), ora.kdata[page][:n_valid, h]), (s, L, h)
                assert np.array_equal(f(v[:n_valid]), ora.vdata[page][:n_valid, h]), (s, L, h)
    qb = W.to_bf16_bits(rng.standard_normal((len(seqs), 8, 128)))
    out, lse = pool.decode(seqs, to_torch(qb, "bf16"), sc.sm_scale)
    torch.cuda.synchronize()
    ro, rl, a, s_abs = att.decode(ora, seqs, f(qb), sc.sm_scale, with_magnitudes=True)
    check_close(out_to_f64(out, "bf16"), ro, BF16_MAX, BF16_MEAN, "decode after kv_append_batch")
    check_close(lse.double().cpu().numpy(), rl, LSE_MAX, LSE_MAX, "decode after kv_append_batch lse")
    check_decode_model(out_to_f64(out, "bf16"), lse.double().cpu().numpy(), ro, rl, a, s_abs, 128, "bf16",
                       "decode after kv_append_batch")
    print("[ok] kv_append_batch", flush=True)


@pytest.mark.parametrize("order", ["copier_first", "writer_first"])
def test_append_batch_rewound_fork_in_shared_tail(order):
    # a has 40 tokens, b = fork(a) rewound to 36 (page 2 shared; a's tokens 36..39 sit in
    # its slots 4..7).  append_batch lists both: whichever comes first copies page 2, the
    # other then owns it alone and writes in place into a slot the copy reads.  Every
    # page's contents must equal the oracle's after the same single appends.
    import torch
    import fork_attention_decode_amd as fa
    from oracle import pagetable as pt
    print(f"[case] kv_append_batch after a rewind into the shared tail ({order})", flush=True)
    hkv, d = 2, 128
    f = W.bf16_bits_to_f64
    rng = np.random.default_rng(17)
    pool = fa.Pool(hkv, d, 16)
    ora = pt.PageTable(16, 16, hkv, d, with_data=True)
    a = pool.seq_create()
    ora.create()
    kb = W.to_bf16_bits(rng.standard_normal((40, hkv, d)) / np.sqrt(d))
    vb = W.to_bf16_bits(rng.standard_normal((40, hkv, d)))
    pool.append(a, to_torch(kb, "bf16"), to_torch(vb, "bf16"))
    ora.append(a, 40, k=f(kb), v=f(vb))
    b = pool.fork(a)
    ora.fork(a)
    pool.rewind(b, 36)
    ora.rewind(b, 36)
    seqs = [a, b] if order == "copier_first" else [b, a]
    for _ in range(3):
        kn = W.to_bf16_bits(rng.standard_normal((2, hkv, d)) / np.sqrt(d))
        vn = W.to_bf16_bits(rng.standard_normal((2, hkv, d)))
        pool.append_batch(seqs, to_torch(kn, "bf16"), to_torch(vn, "bf16"))
        for i, s in enumerate(seqs):
            ora.append(s, 1, k=f(kn[i:i + 1]), v=f(vn[i:i + 1]))
        torch.cuda.synchronize()
    for s in (a, b):
        assert list(pool.block_table(s)) == ora.block_table(s), s
        for L, page in enumerate(ora.block_table(s)):
            n_valid = min(16, ora.seqs[s].n - 16 * L)
            for h in range(hkv):
                k, v = pool.read_page(page, h)
                assert np.array_equal(f(k[:n_valid]), ora.kdata[page][:n_valid, h]), (s, L, h)
                assert np.array_equal(f(v[:n_valid]), ora.vdata[page][:n_valid, h]), (s, L, h)
    print("[ok] kv_append_batch after a rewind into the shared tail", flush=True)


def test_decode_steps_patch_the_plan():
    # decode -> one token appended per branch -> decode ...: once every tail page is owned
    # by its branch alone, each step's plan is patched (tail chunks grow, new pages join the
    # private items) instead of rebuilt; every step against the oracle, and the plan after
    # the last step equals a fresh plan's totals
    import torch
    import fork_attention_decode_amd as fa
    from oracle import attention as att, pagetable as pt
    sc = W.fork_scenario(prefix=517, branches=4, private=[0, 3, 16, 29], hq=8, hkv=2, d=128, seed=41)
    sc.n_pages += 40
    print("[case] decode steps with a patched plan", flush=True)
    pool, _ = build_device_pool(sc)
    ora, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, "bf16"))
    seqs = list(sc.queries)
    f = W.bf16_bits_to_f64
    rng = np.random.default_rng(42)
    patched = 0
    for step in range(37):
        qb = W.to_bf16_bits(rng.standard_normal((len(seqs), 8, 128)))
        out, lse = pool.decode(seqs, to_torch(qb, "bf16"), sc.sm_scale)
        torch.cuda.synchronize()
        patched = max(patched, pool.plan_stats()["patched_changes"])
        ref = att.decode(ora, seqs, f(qb), sc.sm_scale, with_magnitudes=True)
        check_decode_both(out_to_f64(out, "bf16"), lse.double().cpu().numpy(), ref, 128, "bf16", f"step {step}")
        kb = W.to_bf16_bits(rng.standard_normal((len(seqs), 2, 128)) / np.sqrt(128))
        vb = W.to_bf16_bits(rng.standard_normal((len(seqs), 2, 128)))
        pool.append_batch(seqs, to_torch(kb, "bf16"), to_torch(vb, "bf16"))
        for i, b in enumerate(seqs):
            ora.append(b, 1, k=f(kb[i:i + 1]), v=f(vb[i:i + 1]))
    assert patched >= 30, patched
    print(f"[ok] {patched} patched steps; plan {pool.plan_stats()}", flush=True)
