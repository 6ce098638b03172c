"""GPU parity of dag_attn_prefill (block-sparse prefill over the packed DAG mask) against
the fp64 token-level oracle.

Bars: bf16 outputs max-abs 2e-2 and mean-abs 2e-3 against the fp64 oracle, LSE (natural
log, fp32) max-abs 2e-3, and every element within the attention error model's bars
(tests/harness.py: decode_bars; bf16 P, fp32 sums, here with accumulator chains of up to
4,096 steps: gamma = 2^-12, and a row sum over the rounded P).  Small cases compare every row; the full-size packed
workload (81,920 tokens) compares every row of 64 seeded query blocks and of the first and
last block of every segment.
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import check_close, check_decode_model, to_torch

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, LSE_MAX = 2e-2, 2e-3, 2e-3


class _Rows:
    """q in storage dtype, converted to fp64 row by row on access (the oracle only
    touches the rows it is asked for)."""

    def __init__(self, a):
        self.a, self.shape = a, a.shape

    def __getitem__(self, idx):
        return W.bf16_bits_to_f64(self.a[idx])


def _run(pi, label):
    import torch
    import fork_attention_decode_amd as fa
    print(f"[case] {label}: T={pi.T} Hq={pi.n_q_heads} Hkv={pi.n_kv_heads} segments={len(pi.segments)} "
          f"edges={len(pi.edges)}", flush=True)
    mask = fa.DagMask(pi.segments, pi.edges, pi.T, pi.block)
    q, k, v = (to_torch(x, "bf16") for x in (pi.q, pi.k, pi.v))
    out, lse = fa.prefill(q, k, v, mask, pi.sm_scale)
    torch.cuda.synchronize()
    o = W.bf16_bits_to_f64(out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return mask, o, lse.double().cpu().numpy()


def _oracle_rows(pi, rows):
    from oracle import prefill as pf
    k = W.bf16_bits_to_f64(pi.k)
    v = W.bf16_bits_to_f64(pi.v)
    return pf.attend_rows(_Rows(pi.q), k, v, pi.segments, pi.edges, rows, pi.sm_scale, with_magnitudes=True)


def _check(pi, o, lse, rows, label):
    ro, rl, a, s_abs = _oracle_rows(pi, rows)
    mx, mn = check_close(o[rows], ro, BF16_MAX, BF16_MEAN, label)
    check_close(lse[:, rows].T, rl, LSE_MAX, LSE_MAX, label + " lse")
    wo, wl = check_decode_model(o[rows], lse[:, rows].T, ro, rl, a, s_abs, pi.head_dim, "bf16", label,
                                gamma=2.0 ** -12, rounded_p_sum=True)
    print(f"[ok] {label}: {len(rows)} rows, max-abs {mx:.3g} mean-abs {mn:.3g}; error / model bar: O {wo:.3f}, "
          f"LSE {wl:.3f}", flush=True)


@pytest.mark.parametrize("T", [1, 37, 64, 300])
def test_plain_causal(T):
    # one segment, no edges: ordinary causal attention (ragged T, one partial block, T = 1)
    pi = W.prefill_inputs(prefix=T, branches=0, hq=4, hkv=1, seed=31)
    _, o, lse = _run(pi, f"causal T={T}")
    _check(pi, o, lse, list(range(T)), f"causal T={T}")


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
def test_random_dag_shapes(seed):
    # seeded random shapes: prefix, ragged last branch, edges of random length, head
    # counts (G = 1 .. 8); every row is compared
    rng = np.random.default_rng(4000 + seed)
    hq, hkv = [(8, 2), (4, 1), (12, 2), (2, 2), (16, 2)][seed]
    branches = int(rng.integers(1, 6))
    blen = [64 * int(rng.integers(1, 5)) for _ in range(branches - 1)] + [int(rng.integers(1, 300))]
    prefix = 64 * int(rng.integers(1, 5))
    n_edges = int(rng.integers(0, branches * (branches - 1) // 2 + 1))
    pi = W.prefill_inputs(prefix=prefix, branches=branches, branch_len=blen, n_edges=n_edges,
                          edge_len=64 * int(rng.integers(1, 3)), hq=hq, hkv=hkv, seed=40 + seed)
    label = f"random DAG seed={seed} prefix={prefix} branches={blen} edges={n_edges}"
    _, o, lse = _run(pi, label)
    _check(pi, o, lse, list(range(pi.T)), label)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 2), (4, 2), (2, 2), (6, 2), (8, 1)])
def test_small_dag_heads(hq, hkv):
    # G = 4, 8 (two head groups per workgroup set), 2, 1 and 3 (idle waves)
    pi = W.prefill_inputs(prefix=192, branches=3, branch_len=[128, 256, 100], n_edges=3, edge_len=64, hq=hq,
                          hkv=hkv, seed=32)
    _, o, lse = _run(pi, f"small DAG Hq={hq} Hkv={hkv}")
    _check(pi, o, lse, list(range(pi.T)), f"small DAG Hq={hq} Hkv={hkv}")


def test_dag_many_edges_long_rows():
    # 6 branches, every ordered pair an edge: rows reach 10+ column blocks from several sources
    pi = W.prefill_inputs(prefix=640, branches=6, branch_len=[256, 192, 320, 128, 256, 171], n_edges=15,
                          edge_len=128, hq=8, hkv=2, seed=33)
    mask, o, lse = _run(pi, "DAG with 15 edges")
    assert mask.nnz > 0
    _check(pi, o, lse, list(range(pi.T)), "DAG with 15 edges")


def test_packed_dag_full_size():
    """16,384-token prefix + 8 x 8,192 branches, 12 edges of 2,048 tokens (81,920 tokens,
    32 / 8 heads); every row of 64 seeded query blocks and of the first and last block of
    each segment against the oracle, block counts exact."""
    pi = W.dag_prefill()
    mask, o, lse = _run(pi, "packed DAG prefill, full size")
    row_ptr, col, kind = mask.host
    assert mask.nnz == 410240 and int((kind == 1).sum()) == 1280
    rng = np.random.default_rng(7)
    blocks = {int(b) for b in rng.choice(pi.T // 64, size=64, replace=False)}
    for st, ln, _ in pi.segments:
        blocks |= {int(st) // 64, int(st + ln - 1) // 64}
    rows = sorted(r for b in blocks for r in range(64 * b, min(pi.T, 64 * b + 64)))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    _check(pi, o, lse, rows, "packed DAG prefill, full size")


def test_prepare_run_equals_prefill():
    # the two-step form gives the same bits as the one-call form, and a prepared
    # workspace serves a second query set
    import torch
    import fork_attention_decode_amd as fa
    pi = W.prefill_inputs(prefix=192, branches=3, branch_len=[128, 256, 100], n_edges=3, edge_len=64, hq=8, hkv=2,
                          seed=34)
    print("[case] dag_attn_prepare + dag_attn_run == dag_attn_prefill", flush=True)
    mask = fa.DagMask(pi.segments, pi.edges, pi.T, pi.block)
    q, k, v = (to_torch(x, "bf16") for x in (pi.q, pi.k, pi.v))
    o1, l1 = fa.prefill(q, k, v, mask, pi.sm_scale)
    ws = torch.empty(fa.dag_attn_workspace_size(pi.T, 8, 2, 64, mask.nnz), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    fa.dag_attn_prepare(k.data_ptr(), v.data_ptr(), pi.T, 8, 2, 128, mask.row_ptr.data_ptr(), mask.col.data_ptr(),
                        mask.kind.data_ptr(), mask.nnz, 64, ws.data_ptr(), ws.numel(), st)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    q2 = torch.flip(q, dims=[1]).contiguous()
    o3, l3 = torch.empty_like(o1), torch.empty_like(l1)
    for qq, oo, ll in ((q, o2, l2), (q2, o3, l3)):
        fa.dag_attn_run(qq.data_ptr(), oo.data_ptr(), ll.data_ptr(), pi.T, 8, 2, 128, mask.row_ptr.data_ptr(), mask.nnz,
                        64, pi.sm_scale, ws.data_ptr(), ws.numel(), st)
    o4, l4 = fa.prefill(q2, k, v, mask, pi.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
