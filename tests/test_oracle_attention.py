"""Pins for the oracle's decode attention, LSE merge and RoPE (CPU only).

attention: brute force with Python loops, torch's fp64 scaled_dot_product_attention
(a library routine), closed forms (one key, identical keys, zero query), the
grouped-query head map, and equality with naive concatenated-context attention
computed straight from the generator's token blocks (no pool involved).
merge: log-sum-exp merge over random split points equals the unsplit result.
rope: complex-multiplication form, group law R(a)R(b) = R(a+b), inverse, norm
preservation and the relative-position property of dot products.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import workloads as W
from oracle import attention as att, pagetable as pt, rope


def brute(q, k, v, scale):
    s = [scale * sum(q[j] * k[i][j] for j in range(len(q))) for i in range(len(k))]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    o = [sum(e[i] * v[i][j] for i in range(len(k))) / z for j in range(len(v[0]))]
    return o, m + math.log(z)


def test_attend_brute_force():
    rng = np.random.default_rng(1)
    for n in (1, 2, 7, 33):
        q, k, v = rng.standard_normal(5), rng.standard_normal((n, 5)), rng.standard_normal((n, 5))
        o, lse = att.attend(q, k, v, 0.7)
        ob, lb = brute(q.tolist(), k.tolist(), v.tolist(), 0.7)
        assert np.allclose(o, ob, atol=1e-13, rtol=0) and abs(lse - lb) < 1e-13


def test_attend_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(2)
    hq, hkv, n, d = 8, 2, 300, 16
    q = rng.standard_normal((hq, d)); k = rng.standard_normal((n, hkv, d)); v = rng.standard_normal((n, hkv, d))
    o, lse = att.attend_heads(q, k, v, 0.25)
    g = hq // hkv
    kt = torch.from_numpy(np.repeat(k.transpose(1, 0, 2), g, axis=0))[None]   # [1, Hq, n, d]
    vt = torch.from_numpy(np.repeat(v.transpose(1, 0, 2), g, axis=0))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None, :], kt, vt,
                                                           scale=0.25)
    assert np.allclose(o, ref[0, :, 0, :].numpy(), atol=1e-12, rtol=0)
    ref_lse = torch.logsumexp(0.25 * torch.einsum("hd,hnd->hn", torch.from_numpy(q), kt[0]), dim=-1)
    assert np.allclose(lse, ref_lse.numpy(), atol=1e-12, rtol=0)


def test_attend_closed_forms():
    rng = np.random.default_rng(3)
    q, kk, vv = rng.standard_normal(8), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    o, lse = att.attend(q, kk, vv, 0.5)                 # one key: O = v, LSE = s
    assert np.allclose(o, vv[0], atol=1e-15) and abs(lse - 0.5 * q @ kk[0]) < 1e-13
    k = np.tile(kk, (10, 1)); v = rng.standard_normal((10, 8))
    o, lse = att.attend(q, k, v, 0.5)                   # identical keys: mean of V
    assert np.allclose(o, v.mean(0), atol=1e-14) and abs(lse - (0.5 * q @ kk[0] + math.log(10))) < 1e-12
    o, lse = att.attend(np.zeros(8), rng.standard_normal((6, 8)), v[:6], 1.0)   # zero query
    assert np.allclose(o, v[:6].mean(0), atol=1e-14) and abs(lse - math.log(6)) < 1e-13
    o, lse = att.attend(q, np.zeros((0, 8)), np.zeros((0, 8)), 1.0)               # no keys
    assert np.all(o == 0) and lse == -np.inf


def test_gqa_head_map():
    hq, hkv, d, n = 8, 2, 4, 5
    k = np.zeros((n, hkv, d)); v = np.zeros((n, hkv, d))
    v[:, 0, :] = 1.0; v[:, 1, :] = 2.0                  # each KV head has a constant value
    o, _ = att.attend_heads(np.ones((hq, d)), k, v, 1.0)
    assert np.all(o[:4] == 1.0) and np.all(o[4:] == 2.0)   # h // (Hq/Hkv), not h % Hkv


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 80), cuts=st.lists(st.integers(0, 80), max_size=6), seed=st.integers(0, 1000))
def test_lse_merge_invariance(n, cuts, seed):
    rng = np.random.default_rng(seed)
    q, k, v = rng.standard_normal(6), rng.standard_normal((n, 6)) * 3, rng.standard_normal((n, 6))
    pts = sorted(set([0, n] + [c % (n + 1) for c in cuts]))
    parts = [att.partial(q, k[a:b], v[a:b], 0.9) for a, b in zip(pts[:-1], pts[1:])]
    parts.append(att.partial(q, k[:0], v[:0], 0.9))      # an empty piece is skipped
    o, lse = att.merge(parts)
    o2, lse2 = att.attend(q, k, v, 0.9)
    assert np.allclose(o, o2, atol=1e-12, rtol=0) and abs(lse - lse2) < 1e-12


def _naive_context(sc, sid):
    """Visible context of a query sequence straight from the scenario's blocks."""
    f = lambda a: W.storage_to_f64(a, sc.dtype)
    own_k, own_v, mnt = {}, {}, {}
    ids = 0
    for op in sc.ops:
        if op[0] == "create":
            own_k[ids], own_v[ids], mnt[ids] = [], [], []
            ids += 1
        elif op[0] == "fork":
            own_k[ids], own_v[ids], mnt[ids] = list(own_k[op[1]]), list(own_v[op[1]]), list(mnt[op[1]])
            ids += 1
        elif op[0] == "append":
            b = sc.blocks[op[2]]
            own_k[op[1]] += list(f(b.k)); own_v[op[1]] += list(f(b.v))
        elif op[0] == "mount":
            d, s, b, n = op[1:]
            mnt[d] = mnt[d] + list(zip(own_k[s][b:b + n], own_v[s][b:b + n]))
    k = own_k[sid] + [a for a, _ in mnt[sid]]
    v = own_v[sid] + [b for _, b in mnt[sid]]
    return np.stack(k), np.stack(v)


@pytest.mark.parametrize("make", [
    lambda: W.fork_scenario(prefix=50, branches=3, private=[17, 0, 33], hq=4, hkv=2, d=16, seed=5),
    lambda: W.tiny_fork(seed=1),
    lambda: W.dag_scenario(root=64, threads=4, private=48, mounts_per_thread=2, mount_len=20, hq=4, hkv=2,
                           d=16, seed=2),
])
def test_decode_equals_naive_concatenation(make):
    sc = make()
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    table.check_invariants()
    q = W.storage_to_f64(sc.q, sc.dtype)
    o, lse = att.decode(table, sc.queries, q, sc.sm_scale)
    for i, sid in enumerate(sc.queries):
        k, v = _naive_context(sc, sid)
        o2, lse2 = att.attend_heads(q[i], k, v, sc.sm_scale)
        assert np.allclose(o[i], o2, atol=1e-12, rtol=0) and np.allclose(lse[i], lse2, atol=1e-12, rtol=0)


# ------------------------------------------------------------------ rope

def test_rope_complex_form_and_group_law():
    rng = np.random.default_rng(4)
    d, theta = 16, 1e6
    x = rng.standard_normal((5, d))
    delta = np.array([0, 1, -3, 4096, 131071])
    y = rope.rotate(x, delta, theta)
    w = theta ** (-np.arange(d // 2) * 2.0 / d)
    z = (x[:, :d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * delta[:, None] * w[None, :])
    assert np.allclose(y, np.concatenate([z.real, z.imag], 1), atol=1e-12, rtol=0)
    assert np.allclose(rope.rotate(y, -delta, theta), x, atol=1e-9, rtol=0)            # inverse
    a, b = np.array([7, 100, 5000, 1, 0]), np.array([3, -50, 60000, 2, 9])
    assert np.allclose(rope.rotate(rope.rotate(x, a, theta), b, theta), rope.rotate(x, a + b, theta),
                       atol=1e-9, rtol=0)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), atol=1e-12)


def test_rope_relative_position():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(32), rng.standard_normal(32)
    dots = [rope.rotate(q[None], [p + 11], 1e4)[0] @ rope.rotate(k[None], [p], 1e4)[0] for p in (0, 5, 700)]
    assert np.allclose(dots, dots[0], atol=1e-10)


def test_repos_closed_form_from_raw_draws():
    """After drop + repos, the kept key in slot j equals R(j) x / sqrt(d) for the raw fp64
    draw x of that token, up to the one bf16 rounding of the stored key."""
    sc = W.drop_scenario(requests=2, ctx=300, frac=0.4, span_min=20, span_max=50, hq=4, hkv=2, d=32,
                         seed=3, keep_raw=True)
    table, drops = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    table.check_invariants()
    for i in range(2):
        kept = drops[i]
        k, v = table.materialise(i)
        raw = sc.blocks[2 * i].raw_k[kept]
        r = len(kept)
        assert r == 300 - round(0.4 * 300)
        exp = rope.rotate(raw, np.arange(r), sc.rope_theta) / np.sqrt(32)
        assert np.max(np.abs(k[:r] - exp)) < 2 ** -8 * 4 / np.sqrt(32) * 1.01
        assert np.array_equal(v[:r], W.storage_to_f64(sc.blocks[2 * i].v, "bf16")[kept])
        assert list(table.positions(i)) == list(range(r)) + [r]


def test_causal_last_pins():
    # the attention of a sequence's last n tokens (oracle/attention.causal_last):
    # fresh sequence = causal self-attention (torch SDPA, float64); last row = decode;
    # with a mount: own prefix causal and the mounted keys visible to every row
    torch = pytest.importorskip("torch")
    from oracle import attention as att, pagetable as pt
    rng = np.random.default_rng(91)
    hkv, hq, d, P = 2, 4, 8, 4
    t = pt.PageTable(64, P, hkv, d, with_data=True)
    a = t.create()
    k, v = rng.standard_normal((23, hkv, d)), rng.standard_normal((23, hkv, d))
    t.append(a, 23, k=k, v=v)
    q = rng.standard_normal((23, hq, d))
    o, lse = att.causal_last(t, a, q, 0.4)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]                       # [1, Hq, n, d]
    tk = torch.from_numpy(np.repeat(k, hq // hkv, axis=1)).permute(1, 0, 2)[None]
    tv = torch.from_numpy(np.repeat(v, hq // hkv, axis=1)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.4)
    assert np.allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    od, ld = att.decode(t, [a], q[-1:], 0.4)
    assert np.allclose(o[-1], od[0]) and np.allclose(lse[-1], ld[0])
    rows = [22, 0, 7]  # a sample of rows gives those rows of the full result
    os_, ls_ = att.causal_last(t, a, q, 0.4, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls_, lse[rows])
    # mount: b = fork-free second sequence mounting 5 tokens of a
    b = t.create()
    kb, vb = rng.standard_normal((9, hkv, d)), rng.standard_normal((9, hkv, d))
    t.append(b, 9, k=kb, v=vb)
    t.mount(b, a, 3, 5)
    qb = rng.standard_normal((4, hq, d))
    o2, _ = att.causal_last(t, b, qb, 0.4)
    keys = np.concatenate([kb, k[3:8]])
    vals = np.concatenate([vb, v[3:8]])
    for j in range(4):
        vis = np.zeros(len(keys), bool)
        vis[:9 - 4 + j + 1] = True
        vis[9:] = True
        s = torch.einsum("hd,nhd->hn", torch.from_numpy(qb[j]),
                         torch.from_numpy(np.repeat(keys, hq // hkv, axis=1))) * 0.4
        s = s.masked_fill(~torch.from_numpy(vis)[None], float("-inf"))
        want = torch.einsum("hn,nhd->hd", torch.softmax(s, -1), torch.from_numpy(np.repeat(vals, hq // hkv, axis=1)))
        assert np.allclose(o2[j], want.numpy(), rtol=1e-12, atol=1e-12), j
