"""Pins for the packed DAG prefill gradient oracle (CPU only).

- central finite differences of the oracle's own forward loss sum(do * o) on a tiny DAG
  with an edge (pins every term, sign and operand of the three gradients);
- autograd of a dense masked softmax attention in float64 (an independent derivation)
  on a small DAG with grouped heads;
- closed-form invariants: the dS of every row sums to zero, so the dk of each KV head
  sums to zero over the keys, and the dv sums over the keys to the sum of do over the
  group's query heads and rows; a single token has dq = dk = 0 and dv = sum of do;
- the per-row and per-key routines against the full gradients, and the inverse
  visibility rule (seen_by) against the dense token mask.
"""
import numpy as np
import pytest

from oracle import prefill as pf
from oracle import prefill_grad as pg

# tiny DAG: prefix of 4, two branches of 3, an edge exposing 2 tokens of branch 1 to branch 2
SEG = np.array([(0, 4, -1), (4, 3, 0), (7, 3, 0)], np.int32)
EDG = np.array([(1, 1, 2, 2)], np.int32)


def _data(T, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, hq, d)), rng.standard_normal((T, hkv, d)) * 0.7,
            rng.standard_normal((T, hkv, d)), rng.standard_normal((T, hq, d)))


def _loss(q, k, v, do, seg, edg, scale):
    o, _ = pf.attend_rows(q, k, v, seg, edg, range(q.shape[0]), scale)
    return float((o * do).sum())


def test_finite_differences_tiny_dag():
    q, k, v, do = _data(10, 2, 1, 3, 1)
    scale = 0.8
    dq, dk, dv = pg.grads(q, k, v, do, SEG, EDG, scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x[idx] += eps
            lp = _loss(q, k, v, do, SEG, EDG, scale)
            x[idx] -= 2 * eps
            lm = _loss(q, k, v, do, SEG, EDG, scale)
            x[idx] += eps
            num[idx] = (lp - lm) / (2 * eps)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-8), f"d{name}: max diff {np.abs(g - num).max():.3g}"


def test_autograd_dense_masked_attention():
    torch = pytest.importorskip("torch")
    seg = np.array([(0, 9, -1), (9, 7, 0), (16, 8, 0), (24, 6, 1)], np.int32)
    edg = np.array([(1, 2, 3, 2), (2, 0, 4, 3)], np.int32)
    T, hq, hkv, d, scale = 30, 4, 2, 8, 0.35
    q, k, v, do = _data(T, hq, hkv, d, 2)
    mask = torch.from_numpy(pf.visible_mask(seg, edg, T))
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    kx = tk.repeat_interleave(hq // hkv, dim=1)  # [T, Hq, d]
    vx = tv.repeat_interleave(hq // hkv, dim=1)
    s = scale * torch.einsum("ihd,jhd->hij", tq, kx)
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.einsum("hij,jhd->ihd", torch.softmax(s, dim=-1), vx)
    (o * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = pg.grads(q, k, v, do, seg, edg, scale)
    for name, got, ref in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad)):
        assert np.allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12), f"d{name}"


def test_invariants_and_single_token():
    seg = np.array([(0, 20, -1), (20, 12, 0), (32, 9, 0)], np.int32)
    edg = np.array([(1, 4, 5, 2)], np.int32)
    T, hq, hkv, d = 41, 4, 2, 6
    q, k, v, do = _data(T, hq, hkv, d, 3)
    dq, dk, dv = pg.grads(q, k, v, do, seg, edg, 0.5)
    g = hq // hkv
    for h in range(hkv):
        assert np.abs(dk[:, h].sum(axis=0)).max() < 1e-12 * np.abs(dk[:, h]).sum()
        want = do[:, h * g:(h + 1) * g].sum(axis=(0, 1))
        assert np.allclose(dv[:, h].sum(axis=0), want, rtol=1e-12, atol=1e-12)
    one = np.array([(0, 1, -1)], np.int32)
    q1, k1, v1, do1 = _data(1, 4, 2, 5, 4)
    dq1, dk1, dv1 = pg.grads(q1, k1, v1, do1, one, np.zeros((0, 4), np.int32), 0.7)
    assert np.abs(dq1).max() < 1e-15 and np.abs(dk1).max() < 1e-15
    assert np.allclose(dv1[0], do1[0].reshape(2, 2, 5).sum(axis=1))


def test_sampled_routines_match_full_and_seen_by():
    seg = np.array([(0, 16, -1), (16, 10, 0), (26, 9, 0), (35, 7, 0)], np.int32)
    edg = np.array([(1, 2, 4, 2), (1, 6, 3, 3), (2, 0, 5, 3)], np.int32)
    T, hq, hkv, d = 42, 4, 1, 5
    q, k, v, do = _data(T, hq, hkv, d, 5)
    dq, dk, dv = pg.grads(q, k, v, do, seg, edg, 0.6)
    rows = [0, 5, 15, 16, 25, 30, 41]
    _, _, _, mq, mk, mv = pg.grads(q, k, v, do, seg, edg, 0.6, magnitudes=True)
    rq, rmq = pg.dq_rows(q, k, v, do, seg, edg, 0.6, rows)
    assert np.allclose(rq, dq[rows], rtol=1e-12, atol=1e-14) and np.allclose(rmq, mq[rows], rtol=1e-12)
    keys = [0, 15, 17, 19, 22, 26, 31, 41]
    sk, sv, smk, smv = pg.dkdv_keys(q, k, v, do, seg, edg, 0.6, keys)
    assert np.allclose(sk, dk[keys], rtol=1e-12, atol=1e-14)
    assert np.allclose(sv, dv[keys], rtol=1e-12, atol=1e-14)
    assert np.allclose(smk, mk[keys], rtol=1e-12) and np.allclose(smv, mv[keys], rtol=1e-12)
    # a magnitude bounds its gradient
    assert np.all(np.abs(dq) <= mq + 1e-12) and np.all(np.abs(dk) <= mk + 1e-12) and np.all(np.abs(dv) <= mv + 1e-12)
    dense = pf.visible_mask(seg, edg, T)
    for j in range(T):
        assert np.array_equal(pg.seen_by(seg, edg, T, j), np.nonzero(dense[:, j])[0]), j
