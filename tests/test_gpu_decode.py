"""GPU parity of fork_attn_decode (HIP path through the C ABI) against the fp64 oracle.

Tolerances: bf16 outputs max-abs 2e-2 and mean-abs 2e-3 against the fp64 oracle
(fp32 accumulation in the kernels); fp32 pools max-abs 1e-4; LSE (fp32) max-abs 2e-3.
Integer state (block tables, refcounts) bit-exact.  Every case prints its name first.
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import build_device_pool, check_close, oracle_decode, out_to_f64, subscenario, to_torch

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX, LSE_MAX = 2e-2, 2e-3, 1e-4, 2e-3


def _run(sc, label):
    import torch
    print(f"[case] {label}: {sc.name} Hq={sc.n_q_heads} Hkv={sc.n_kv_heads} d={sc.head_dim} {sc.dtype}", flush=True)
    pool, _ = build_device_pool(sc)
    q = to_torch(sc.q, sc.dtype)
    out, lse = pool.decode(sc.queries, q, sc.sm_scale)
    torch.cuda.synchronize()
    return pool, out_to_f64(out, sc.dtype), lse.double().cpu().numpy()


def _check(sc, o, lse, label, rows=None):
    ro, rl = oracle_decode(sc, rows)
    if rows is not None:
        o, lse = o[rows], lse[rows]
    if sc.dtype == "bf16":
        mx, mn = check_close(o, ro, BF16_MAX, BF16_MEAN, label)
    else:
        mx, mn = check_close(o, ro, F32_MAX, F32_MAX, label)
    check_close(lse, rl, LSE_MAX, LSE_MAX, label + " lse")
    print(f"[ok] {label}: max-abs {mx:.3g} mean-abs {mn:.3g}", flush=True)


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
    assert pool.plan_stats()["unique_kv_bytes"] == 536870912
    _check(sc, o, lse, "Octopus DAG decode, full size")


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
    ro, rl = att.decode(ora, seqs, f(qb), sc.sm_scale)
    check_close(out_to_f64(out, "bf16"), ro, BF16_MAX, BF16_MEAN, "decode after kv_append_batch")
    check_close(lse.double().cpu().numpy(), rl, LSE_MAX, LSE_MAX, "decode after kv_append_batch lse")
    print("[ok] kv_append_batch", flush=True)
