"""GPU parity of kv_drop / kv_repos (fused compaction + re-rotation kernel) and of decode
over compacted sequences, against the fp64 oracle.

Bars: block tables, positions, refcounts and free counts bit-exact; V moved bit-exactly;
K without repos bit-exact; re-rotated K within one bf16 ulp of the oracle's fp64 rotation
of the stored key (plus 4e-7 x the pair's magnitude for the fp32 products); decode
outputs as in the other decode tests (bf16 max-abs 2e-2 / mean-abs 2e-3, LSE 2e-3) and
within the decode error model's bars, whose score term includes one bf16 ulp of every
re-rotated key (tests/harness.py: decode_bars).  The full-size case also plants one key
per row of the two checked requests (the row's output is then that key's value).
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import (build_device_pool, check_close, check_decode_both, check_decode_model, oracle_decode,
                           out_to_f64,
                           plant_queries, subscenario, to_torch)

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, LSE_MAX = 2e-2, 2e-3, 2e-3


def _oracle(sc):
    from oracle import pagetable as pt
    return pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))


def _k_close(got_st, ref, what, dtype="bf16"):
    """got_st: keys in storage form [n, d] (bf16 bits or fp32); ref: fp64 [n, d].  One ulp
    of the reference value in the storage type, plus the fp32 product error of a rotation of
    the pair (x_i, x_{i+d/2})."""
    got = W.storage_to_f64(got_st, dtype)
    _, e = np.frexp(ref)
    ulp = np.ldexp(1.0, e - (8 if dtype == "bf16" else 24))
    h = ref.shape[-1] // 2
    pair = np.abs(ref) + np.abs(np.concatenate([ref[..., h:], ref[..., :h]], axis=-1))
    bad = np.abs(got - ref) > ulp + 4e-7 * pair
    assert not bad.any(), f"{what}: {int(bad.sum())} keys off by more than one ulp, e.g. {got[bad][:4]} vs {ref[bad][:4]}"


def _check_state(sc, pool, ora, seqs, pages=None, exact_k=None):
    """Integer state of `seqs` bit-exact; page contents of every valid slot (or of the listed
    logical pages)."""
    for s in seqs:
        bt = ora.block_table(s)
        assert list(pool.block_table(s)) == bt, f"block table of sequence {s}"
        assert np.array_equal(pool.positions(s), ora.positions(s)), f"positions of sequence {s}"
        n = ora.seqs[s].n
        for L in (range(len(bt)) if pages is None else pages):
            page = bt[L]
            nv = min(16, n - 16 * L)
            for h in range(sc.n_kv_heads):
                k, v = pool.read_page(page, h)
                rk, rv = ora.kdata[page][:nv, h], ora.vdata[page][:nv, h]
                assert np.array_equal(W.storage_to_f64(v[:nv], sc.dtype), rv), f"V of seq {s} page {L} head {h}"
                if exact_k is not None and exact_k(s):
                    assert np.array_equal(W.storage_to_f64(k[:nv], sc.dtype), rk), f"K of seq {s} page {L} head {h}"
                else:
                    _k_close(k[:nv], rk, f"K of seq {s} page {L} head {h}", sc.dtype)
    assert pool.free_pages() == ora.n_free
    for p in range(sc.n_pages):
        assert pool.refcount(p) == ora.rc[p], f"refcount of page {p}"
    assert pool.sync_status() == 0, "compaction ordering waits timed out"


@pytest.mark.parametrize("repos", [True, False])
def test_drop_compaction_contents(repos):
    sc = W.drop_scenario(requests=2, ctx=1000, frac=0.4, span_min=17, span_max=150, hq=4, hkv=2, d=128,
                         seed=21, repos=repos)
    print(f"[case] drop contents repos={repos}: {[op[2] for op in sc.ops if op[0] == 'drop']}", flush=True)
    pool, kept = build_device_pool(sc)
    ora, okept = _oracle(sc)
    for a, b in zip(kept, okept):
        assert np.array_equal(a, b)
    _check_state(sc, pool, ora, [0, 1], exact_k=lambda s: not repos)


@pytest.mark.parametrize("dtype,d", [("fp32", 128), ("bf16", 64), ("fp32", 64)])
def test_drop_repos_other_storage(dtype, d):
    # the compaction kernel's other instantiations: fp32 pools (one slot per 32-bit word of a
    # V^T row, no half-word shifts) and head dim 64; page contents, then a decode
    import torch
    sc = W.drop_scenario(requests=2, ctx=900, frac=0.4, span_min=17, span_max=150, hq=4, hkv=2, d=d, dtype=dtype,
                         seed=27, repos=True)
    print(f"[case] drop + repos, {dtype} d={d}", flush=True)
    pool, kept = build_device_pool(sc)
    ora, okept = _oracle(sc)
    for a, b in zip(kept, okept):
        assert np.array_equal(a, b)
    _check_state(sc, pool, ora, [0, 1])
    out, lse = pool.decode(sc.queries, to_torch(sc.q, dtype), sc.sm_scale)
    torch.cuda.synchronize()
    mx, mn, _, _ = check_decode_both(out_to_f64(out, dtype), lse.double().cpu().numpy(),
                                     oracle_decode(sc, with_magnitudes=True), d, dtype,
                                     f"decode after drop {dtype} d={d}", rerotated_keys=True)
    print(f"[ok] max-abs {mx:.3g} mean-abs {mn:.3g}", flush=True)


def test_drop_many_offsets_and_edge_spans():
    # single-token spans every 7 tokens (hundreds of distinct repos offsets), a drop of
    # the tail only, a drop of nothing, and a drop of everything
    n = 3000
    sc = W.drop_scenario(requests=4, ctx=n, frac=0.0, hq=4, hkv=2, d=128, seed=22, repos=True)
    spans = {0: [(t, 1) for t in range(3, n, 7)], 1: [(n - 37, 37)], 2: [], 3: [(0, n)]}
    ops = []
    for op in sc.ops:
        if op[0] == "drop":
            ops.append(("drop", op[1], spans[op[1]], True))
        elif op[0] == "append" and sc.blocks[op[2]].pos.shape[0] == 1:
            continue  # no decode token: positions of the sequences are checked directly
        else:
            ops.append(op)
    sc.ops = ops
    print("[case] drop with 429 distinct offsets / tail only / nothing / everything", flush=True)
    pool, _ = build_device_pool(sc)
    ora, _ = _oracle(sc)
    _check_state(sc, pool, ora, [0, 1, 2, 3])


def test_drop_on_shared_pages_cow():
    # forks share the prefix: a drop in a fork copies the shared pages it rewrites and
    # leaves the root's pages untouched
    sc = W.fork_scenario(prefix=517, branches=3, private=[60, 200, 9], hq=4, hkv=2, d=128, seed=23)
    sc.ops = sc.ops + [("drop", 1, [(40, 33), (300, 100)], True), ("drop", 2, [(600, 50)], False),
                       ("drop", 3, [(0, 5)], True)]
    sc.n_pages += 120  # room for the copies
    print("[case] drop on forks sharing a prefix (copy-on-write)", flush=True)
    pool, _ = build_device_pool(sc)
    ora, _ = _oracle(sc)
    _check_state(sc, pool, ora, [0, 1, 2, 3], exact_k=lambda s: s in (0, 2))


def test_drop_on_mounted_sequence():
    # thread pages mounted by siblings stay referenced: the drop copies them
    sc = W.dag_scenario(root=300, threads=4, private=200, mounts_per_thread=2, mount_len=70, hq=8, hkv=2, d=128,
                        seed=24)
    sc.ops = sc.ops + [("drop", 1, [(10, 20), (350, 64)], True), ("drop", 2, [(299, 100)], True)]
    sc.n_pages += 80  # room for the copies
    print("[case] drop on a mounted DAG thread", flush=True)
    pool, _ = build_device_pool(sc)
    ora, _ = _oracle(sc)
    _check_state(sc, pool, ora, list(range(5)), exact_k=lambda s: s not in (1, 2))
    import torch
    q = to_torch(sc.q, sc.dtype)
    out, lse = pool.decode(sc.queries, q, sc.sm_scale)
    torch.cuda.synchronize()
    check_decode_both(out_to_f64(out, "bf16"), lse.double().cpu().numpy(), oracle_decode(sc, with_magnitudes=True),
                      128, "bf16", "decode after drop on mounted thread", rerotated_keys=True)


@pytest.mark.parametrize("repos", [True, False])
def test_decode_after_drop(repos):
    import torch
    sc = W.drop_scenario(requests=3, ctx=5000, frac=0.4, span_min=64, span_max=700, hq=8, hkv=2, d=128,
                         seed=25, repos=repos)
    print(f"[case] decode after drop repos={repos}", flush=True)
    pool, _ = build_device_pool(sc)
    q = to_torch(sc.q, sc.dtype)
    out, lse = pool.decode(sc.queries, q, sc.sm_scale)
    torch.cuda.synchronize()
    mx, mn, wo, wl = check_decode_both(out_to_f64(out, "bf16"), lse.double().cpu().numpy(),
                                       oracle_decode(sc, with_magnitudes=True), 128, "bf16", "decode after drop",
                                       rerotated_keys=repos)
    print(f"[ok] max-abs {mx:.3g} mean-abs {mn:.3g}; error / model bar: O {wo:.3f}, LSE {wl:.3f}", flush=True)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_drops(seed):
    # seeded random shapes: request count, context length, dropped fraction and span
    # lengths, repos or not; page contents, tables and counts exact, then a decode
    import torch
    rng = np.random.default_rng(5000 + seed)
    repos = bool(seed % 2)
    ctx = int(rng.integers(20, 2500))
    sc = W.drop_scenario(requests=int(rng.integers(1, 4)), ctx=ctx, frac=float(rng.uniform(0.05, 0.9)),
                         span_min=int(rng.integers(1, 20)), span_max=int(rng.integers(20, 300)), hq=8, hkv=2, d=128,
                         seed=50 + seed, repos=repos)
    print(f"[case] random drops seed={seed} ctx={ctx} repos={repos}: "
          f"{[op[2] for op in sc.ops if op[0] == 'drop']}", flush=True)
    pool, kept = build_device_pool(sc)
    ora, okept = _oracle(sc)
    for a, b in zip(kept, okept):
        assert np.array_equal(a, b)
    _check_state(sc, pool, ora, sorted(set(sc.queries)), exact_k=lambda s: not repos)
    out, lse = pool.decode(sc.queries, to_torch(sc.q, sc.dtype), sc.sm_scale)
    torch.cuda.synchronize()
    mx, mn, wo, wl = check_decode_both(out_to_f64(out, "bf16"), lse.double().cpu().numpy(),
                                       oracle_decode(sc, with_magnitudes=True), 128, "bf16",
                                       f"decode after random drops seed={seed}", rerotated_keys=repos)
    print(f"[ok] max-abs {mx:.3g} mean-abs {mn:.3g}; error / model bar: O {wo:.3f}, LSE {wl:.3f}", flush=True)


def test_akv_drop_repos_full_size():
    """16 requests x 131,072 tokens, 40 % dropped, repos, decode; the oracle checks two
    sampled requests end to end (page table, sampled pages, decode output)."""
    import torch
    sc = W.akv_drop_repos()
    print("[case] AKV drop + repos + decode, full size (16 x 131,072)", flush=True)
    pool, kept = build_device_pool(sc)
    q = to_torch(sc.q, sc.dtype)
    out, lse = pool.decode(sc.queries, q, sc.sm_scale)
    torch.cuda.synchronize()
    assert pool.sync_status() == 0
    o = out_to_f64(out, "bf16")
    l = lse.double().cpu().numpy()
    for req in (0, 11):
        sub = subscenario(sc, [req])
        ora, okept = _oracle(sub)
        assert np.array_equal(kept[req], okept[0])
        bt = ora.block_table(0)
        assert list(pool.block_table(req)) != [] and len(pool.block_table(req)) == len(bt)
        assert np.array_equal(pool.positions(req), ora.positions(0))
        # sampled pages: first, a few inside, the last (with the decode token)
        own = pool.block_table(req)
        for L in sorted({0, 1, len(bt) // 3, len(bt) // 2, len(bt) - 2, len(bt) - 1}):
            nv = min(16, ora.seqs[0].n - 16 * L)
            for h in (0, 5):
                k, v = pool.read_page(int(own[L]), h)
                assert np.array_equal(W.bf16_bits_to_f64(v[:nv]), ora.vdata[bt[L]][:nv, h])
                _k_close(k[:nv], ora.kdata[bt[L]][:nv, h], f"request {req} page {L} head {h}")
        mx, mn, wo, wl = check_decode_both(o[[req]], l[[req]], oracle_decode(sub, with_magnitudes=True), 128, "bf16",
                                           f"request {req}", rerotated_keys=True)
        print(f"[ok] request {req}: max-abs {mx:.3g} mean-abs {mn:.3g}; error / model bar: O {wo:.3f}, "
              f"LSE {wl:.3f}", flush=True)
    # planted keys: rows of requests 0 and 11 single out one key each (drawn from the
    # oracle's compacted context); the other requests keep their queries
    qp = sc.q.copy()
    planted = {}
    for req in (0, 11):
        sub = subscenario(sc, [req])
        qs, vp, _ = plant_queries(sub, np.random.default_rng(100 + req))
        qp[req] = qs[0]
        planted[req] = (sub, qs, vp)
    out, lse = pool.decode(sc.queries, to_torch(qp, sc.dtype), sc.sm_scale)
    torch.cuda.synchronize()
    o = out_to_f64(out, "bf16")
    l = lse.double().cpu().numpy()
    for req, (sub, qs, vp) in planted.items():
        bad = np.abs(o[req] - vp[0]) > 2.0 ** -8 * np.abs(vp[0]) + 1e-6
        assert not bad.any(), f"planted keys of request {req}: {int(bad.sum())} elements differ from v_j"
        # planted scores are ~40: the keys' one-ulp rounding moves them by up to 2^-7 x 40,
        # so only the error model (which scales with the scores) applies, not the fixed
        # 2e-3 LSE gate
        ro, rl, a, s_abs = oracle_decode(sub, with_magnitudes=True, q=qs)
        check_decode_model(o[[req]], l[[req]], ro, rl, a, s_abs, 128, "bf16", f"planted keys, request {req}",
                           rerotated_keys=True)
    print("[ok] planted keys of requests 0 and 11", flush=True)


@pytest.mark.parametrize("shared", [False, True])
def test_drop_batch_contents(shared):
    # kv_drop_batch against the oracle's drops one after another in list order: independent
    # requests (one launch), or forks sharing a prefix whose copies land on pages an
    # earlier drop of the list released while still reading them (split launches)
    import torch
    if shared:
        sc = W.fork_scenario(prefix=517, branches=3, private=[160, 300, 90], hq=4, hkv=2, d=128, seed=95)
        sc.n_pages += 120
        seqs = [2, 1, 3]
        spans = [[(40, 33), (300, 100)], [(0, 5), (500, 20)], [(600, 7)]]
    else:
        sc = W.drop_scenario(requests=4, ctx=1100, frac=0.0, hq=4, hkv=2, d=128, seed=96, repos=True)
        sc.ops = [op for op in sc.ops if op[0] != "drop" and not (op[0] == "append" and len(sc.blocks[op[2]].pos) == 1)]
        seqs = [3, 0, 2, 1]
        spans = [[(17, 300), (700, 64)], [(0, 16)], [], [(1000, 100)]]
    print(f"[case] kv_drop_batch shared={shared}: {list(zip(seqs, spans))}", flush=True)
    pool, _ = build_device_pool(sc)
    ora, _ = _oracle(sc)
    kept = pool.drop_batch(seqs, spans, repos=True)
    torch.cuda.synchronize()
    for s, sp, k in zip(seqs, spans, kept):
        assert np.array_equal(k, ora.drop(s, sp, repos=True)), s
    live = [i for i, s in enumerate(ora.seqs) if s.live]
    _check_state(sc, pool, ora, live, exact_k=lambda s: s not in seqs)
    print("[ok] kv_drop_batch", flush=True)
