"""GPU parity of dag_attn_backward (gradients of the block-sparse prefill over the packed
DAG mask) against the fp64 gradient oracle (oracle/prefill_grad.py).

Both sides take the same bf16 q, k, v and upstream gradient dout; the library also takes
its own forward's bf16 out and fp32 lse, the oracle recomputes them in fp64.

Bars, per element: |got - ref| <= 2^-7 x magnitude + 1e-4 x RMS, where the magnitude is
the same sum over the magnitudes of its terms (oracle/prefill_grad.py).  The library
rounds P and dS to bf16 before the products over queries (dV, dK) and keys (dQ): at
most 2^-8 relative in every term, so at most 2^-8 x magnitude in the sum; D = dout.out
uses the bf16 forward output (2^-9 relative, inside the magnitude's P_ij d_i part); the
fp32 dot products and exponentials add ~1e-5 relative.  The bar takes twice the bf16
bound.  And on the whole tensor: mean-abs <= 4e-3 x RMS (about 2^-8 / sqrt(3) = 2.3e-3
is expected from random-signed roundings; the RMS is floored at 1e-3 -- dout is N(0, 1)
-- for tensors that are zero in exact arithmetic, like dq and dk of a single token).
Small cases compare every element; the full-size
packed workload (81,920 tokens) compares sampled dq rows, the dk / dv of the last keys
of the last branch (whose readers are few), and two sums that hold at any size: over
the keys of a KV head, dv sums to the sum of dout over its query heads and rows, and dk
sums to zero (every row of dS sums to zero).
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import to_torch

pytestmark = pytest.mark.gpu

MEAN_REL = 4e-3


def _dout(pi, seed):
    return W.to_bf16_bits(np.random.default_rng(seed).standard_normal((pi.T, pi.n_q_heads, pi.head_dim)))


def _run(pi, dob, label):
    import torch
    import fork_attention_decode_amd as fa
    print(f"[case] {label}: T={pi.T} Hq={pi.n_q_heads} Hkv={pi.n_kv_heads} segments={len(pi.segments)} "
          f"edges={len(pi.edges)}", flush=True)
    mask = fa.DagMask(pi.segments, pi.edges, pi.T, pi.block)
    q, k, v, do = (to_torch(x, "bf16") for x in (pi.q, pi.k, pi.v, dob))
    out, lse = fa.prefill(q, k, v, mask, pi.sm_scale)
    dq, dk, dv = fa.prefill_backward(q, k, v, out, do, lse, mask, pi.sm_scale)
    torch.cuda.synchronize()
    return mask, dq.double().cpu().numpy(), dk.double().cpu().numpy(), dv.double().cpu().numpy()


def _close(got, ref, mag, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    rms = max(float(np.sqrt(np.mean(ref ** 2))), 1e-3)  # floor: tensors that are zero in exact arithmetic
    err = np.abs(got - ref)
    ratio = err / (2.0 ** -7 * mag + 1e-4 * rms)
    worst, mn = float(ratio.max()), float(err.mean())
    assert worst <= 1.0 and mn <= MEAN_REL * rms, \
        f"{what}: worst error / bar {worst:.3g}, mean-abs {mn:.3g} vs RMS {rms:.3g} ({mn / rms:.3g})"
    print(f"[ok] {what}: worst error / bar {worst:.3g}, max-abs {float(err.max()) / rms:.3g} and mean-abs "
          f"{mn / rms:.3g} of RMS {rms:.3g}", flush=True)


def _full_check(pi, seed, label):
    from oracle import prefill_grad as pg
    dob = _dout(pi, seed)
    _, dq, dk, dv = _run(pi, dob, label)
    f = W.bf16_bits_to_f64
    rq, rk, rv, mq, mk, mv = pg.grads(f(pi.q), f(pi.k), f(pi.v), f(dob), pi.segments, pi.edges, pi.sm_scale,
                                      magnitudes=True)
    _close(dq, rq, mq, label + " dq")
    _close(dk, rk, mk, label + " dk")
    _close(dv, rv, mv, label + " dv")


@pytest.mark.parametrize("T", [1, 37, 64, 300])
def test_plain_causal(T):
    # one segment, no edges: causal attention's gradients (ragged T, one partial block, T = 1)
    pi = W.prefill_inputs(prefix=T, branches=0, hq=4, hkv=1, seed=61)
    _full_check(pi, 62, f"backward causal T={T}")


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 2), (2, 2), (6, 2), (8, 1)])
def test_small_dag_heads(hq, hkv):
    # G = 4, 2, 1, 3 (odd: one head per dQ workgroup) and 8; ragged last branch, 3 edges
    pi = W.prefill_inputs(prefix=192, branches=3, branch_len=[128, 256, 100], n_edges=3, edge_len=64, hq=hq,
                          hkv=hkv, seed=63)
    _full_check(pi, 64, f"backward small DAG Hq={hq} Hkv={hkv}")


def test_dag_many_edges():
    # 5 branches, every ordered pair an edge: key blocks read by many query blocks
    pi = W.prefill_inputs(prefix=320, branches=5, branch_len=[192, 128, 256, 128, 75], n_edges=10, edge_len=64,
                          hq=8, hkv=2, seed=65)
    _full_check(pi, 66, "backward DAG with 10 edges")


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
def test_random_dag_shapes(seed):
    # seeded random shapes: prefix, ragged last branch, edges, head counts (G = 1 .. 8); the
    # key-block pairs, the head pairs of the dK/dV stages and the packed rows of the dQ pass
    # all see uneven counts
    rng = np.random.default_rng(1000 + seed)
    hq, hkv = [(4, 1), (8, 2), (6, 2), (2, 2), (8, 1)][seed]
    branches = int(rng.integers(1, 5))
    blen = [64 * int(rng.integers(1, 4)) for _ in range(branches - 1)] + [int(rng.integers(1, 200))]
    prefix = 64 * int(rng.integers(1, 4))
    n_edges = int(rng.integers(0, branches * (branches - 1) // 2 + 1))
    pi = W.prefill_inputs(prefix=prefix, branches=branches, branch_len=blen, n_edges=n_edges, edge_len=64, hq=hq,
                          hkv=hkv, seed=70 + seed)
    _full_check(pi, 80 + seed, f"backward random DAG seed={seed} prefix={prefix} branches={blen} "
                               f"edges={n_edges} Hq={hq} Hkv={hkv}")


def test_skipped_columns_change_nothing():
    # entries whose column is outside [0, nb) are skipped: the same mask with such entries
    # added at the ends of some rows (kept ascending, some marked diagonal) gives the same
    # gradients, bit for bit
    import torch
    import fork_attention_decode_amd as fa
    from types import SimpleNamespace
    pi = W.prefill_inputs(prefix=192, branches=3, branch_len=[128, 256, 100], n_edges=3, edge_len=64, hq=8,
                          hkv=2, seed=68)
    dob = _dout(pi, 69)
    mask = fa.DagMask(pi.segments, pi.edges, pi.T, pi.block)
    q, k, v, do = (to_torch(x, "bf16") for x in (pi.q, pi.k, pi.v, dob))
    out, lse = fa.prefill(q, k, v, mask, pi.sm_scale)
    ref = fa.prefill_backward(q, k, v, out, do, lse, mask, pi.sm_scale)
    row_ptr, col, kind = mask.host
    nb = len(row_ptr) - 1
    rp, cols, kinds = [0], [], []
    for r in range(nb):
        c, kd = list(col[row_ptr[r]:row_ptr[r + 1]]), list(kind[row_ptr[r]:row_ptr[r + 1]])
        if r % 2 == 0:
            c, kd = [-1 - r] + c, [1] + kd
        if r % 3 == 0:
            c, kd = c + [nb, nb + 7], kd + [0, 1]
        cols += c
        kinds += kd
        rp.append(len(cols))
    print(f"[case] skipped columns: nb={nb}, nnz {mask.nnz} -> {len(cols)}", flush=True)
    padded = SimpleNamespace(T=mask.T, block=mask.block, nnz=len(cols),
                             row_ptr=torch.tensor(rp, dtype=torch.int32, device="cuda"),
                             col=torch.tensor(cols, dtype=torch.int32, device="cuda"),
                             kind=torch.tensor(kinds, dtype=torch.uint8, device="cuda"))
    got = fa.prefill_backward(q, k, v, out, do, lse, padded, pi.sm_scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), f"{name} differs with skipped entries"


def test_packed_dag_full_size():
    """81,920 tokens, 32 / 8 heads: sampled dq rows and last-branch keys against the
    oracle, and the two sums over all keys."""
    from oracle import prefill_grad as pg
    pi = W.dag_prefill()
    dob = _dout(pi, 67)
    mask, dq, dk, dv = _run(pi, dob, "backward packed DAG, full size")
    assert mask.nnz == 410240
    f = W.bf16_bits_to_f64
    k, v = f(pi.k), f(pi.v)

    class Rows:  # q and dout converted row by row on access
        def __init__(self, a):
            self.a, self.shape = a, a.shape

        def __getitem__(self, idx):
            return f(self.a[idx])

    q, do = Rows(pi.q), Rows(dob)
    rows = sorted({int(st) for st, _, _ in pi.segments} | {int(st + ln - 1) for st, ln, _ in pi.segments}
                  | {int(pi.segments[dst][0]) + 64 for _, _, _, dst in pi.edges[:4]})
    print(f"[case] full size: {len(rows)} dq rows", flush=True)
    rq, mq = pg.dq_rows(q, k, v, do, pi.segments, pi.edges, pi.sm_scale, rows)
    _close(dq[rows], rq, mq, "full size dq rows")
    keys = list(range(pi.T - 12, pi.T))  # the last branch is no edge's source: few readers
    print(f"[case] full size: dk / dv of keys {keys[0]}..{keys[-1]}", flush=True)
    rk, rv, mk, mv = pg.dkdv_keys(q, k, v, do, pi.segments, pi.edges, pi.sm_scale, keys)
    _close(dk[keys], rk, mk, "full size dk keys")
    _close(dv[keys], rv, mv, "full size dv keys")
    g = pi.n_q_heads // pi.n_kv_heads
    dsum = f(dob).reshape(pi.T, pi.n_kv_heads, g, pi.head_dim).sum(axis=(0, 2))
    assert np.allclose(dv.sum(axis=0), dsum, rtol=0, atol=2e-3 * np.abs(dsum).max() + 1e-3), "sum of dv"
    ksum = np.abs(dk.sum(axis=0)).max()
    assert ksum <= 1e-3 * np.abs(dk).sum(axis=0).max(), f"sum of dk {ksum:.3g}"
    print("[ok] full size sums", flush=True)
