"""Shared helpers of the GPU parity tests and the bench: replay a ``workloads`` scenario
through the library on the device, and through the oracle on the CPU."""
from __future__ import annotations

import numpy as np

import workloads as W


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def out_to_f64(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return W.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


def build_device_pool(sc: W.Scenario, extra_pages: int = 0, stream_sync: bool = True):
    """Replay the scenario's operations on a device pool.  Returns (pool, kept lists)."""
    import torch
    import fork_attention_decode_amd as fa
    pool = fa.Pool(sc.n_kv_heads, sc.head_dim, sc.n_pages + extra_pages, dtype=sc.dtype,
                   rope_theta=sc.rope_theta)
    kept = []
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "append":
            blk = sc.blocks[op[2]]
            k = to_torch(blk.k, sc.dtype)
            v = to_torch(blk.v, sc.dtype)
            pool.append(op[1], k, v, positions=blk.pos)
            if stream_sync:
                torch.cuda.synchronize()  # keep k / v alive until the copy kernel ran
        elif op[0] == "fork":
            pool.fork(op[1])
        elif op[0] == "mount":
            pool.mount(*op[1:])
        elif op[0] == "drop":
            kept.append(pool.drop(op[1], op[2], repos=op[3]))
        elif op[0] == "release":
            pool.release(op[1])
    torch.cuda.synchronize()
    return pool, kept


def oracle_decode(sc: W.Scenario, rows=None, with_magnitudes: bool = False, q=None):
    """fp64 oracle outputs (o [n, Hq, d], lse [n, Hq]) for the scenario's queries (or the
    listed query indices); with_magnitudes adds the error-model terms (a, s_abs) of
    ``oracle.attention.magnitudes``.  q: storage-form queries replacing sc.q."""
    from oracle import attention as att, pagetable as pt
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    q = W.storage_to_f64(sc.q if q is None else q, sc.dtype)
    idx = list(range(len(sc.queries))) if rows is None else list(rows)
    return att.decode(table, [sc.queries[i] for i in idx], q[idx], sc.sm_scale, with_magnitudes=with_magnitudes)


# ---------------------------------------------------------------- decode error model
# Bars for a decode output against the fp64 oracle, derived from the kernel's arithmetic
# (not from observed errors).  Per row: n visible keys, softmax weights pi_j, a_e =
# sum_j pi_j |v_je| and S = scale * max_j sum_i |q_i k_ji| (oracle.attention.magnitudes).
#   scores   bf16 x bf16 products are exact in fp32, the d-term sum and the two scalings
#            (scale, log2 e) round at most d + 2 times: |ds| <= eps_s = (d + 2) 2^-24 S;
#            keys re-rotated by Repos are stored rounded to the pool type, within one
#            ulp (2^-7 relative for bf16, 2^-23 for fp32) of the oracle's fp64
#            rotation: + 2^-7 S (bf16) or 2^-23 S (fp32);
#   weights  a score error moves pi_j by at most a factor exp(+-2 eps_s);
#   P        p_j is rounded to bf16 (RNE, unit roundoff 2^-8) before the P V product; the
#            decode's normaliser l sums the unrounded p: |dO_e| <= 2^-8 a_e; the prefill's
#            sums the rounded p (rounded_p_sum): |dO_e| <= 2^-8 (a_e + |O_e|) and the
#            lse moves by up to 2^-8 more;
#   sums     every fp32 accumulator chain (l, the P V accumulators, the merge) has at
#            most 512 roundings: gamma = 2^-15 relative (2^-13 for fp32 pools, whose
#            16x16x4 products take 8x more steps);
#   output   rounded to the pool type: 2^-8 |O_e| (bf16), 2^-24 (fp32);
#   lse      |dlse| <= eps_s + gamma + 2^-22 |lse| (the log2 -> ln conversion).
# So |dO_e| <= 2^-8 a_e [bf16] + expm1(2 eps_s) a_e + gamma a_e + u_out |O_e| + 1e-7.
def decode_bars(ref_o, ref_lse, a, s_abs, head_dim: int, dtype: str, rerotated_keys: bool = False,
                gamma: float = None, rounded_p_sum: bool = False):
    """gamma: relative bound of the fp32 accumulator chains when longer than the split-K
    decode's (the prefill's P V accumulators step 16 keys at a time over a whole row)."""
    d = head_dim
    key_ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -23  # one ulp of a stored re-rotated key, relative
    eps_s = (d + 2) * 2.0 ** -24 * s_abs + (key_ulp * s_abs if rerotated_keys else 0.0)
    if gamma is None:
        gamma = 2.0 ** -15 if dtype == "bf16" else 2.0 ** -13
    u_p = 2.0 ** -8 if dtype == "bf16" else 0.0
    u_out = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    bar_o = (u_p + np.expm1(2 * eps_s)[..., None] + gamma) * a + (u_out + (u_p if rounded_p_sum else 0.0)) * np.abs(
        ref_o) + 1e-7
    bar_lse = eps_s + gamma + 2.0 ** -22 * np.abs(ref_lse) + (u_p if rounded_p_sum else 0.0)
    return bar_o, bar_lse


def check_decode_model(o, lse, ref_o, ref_lse, a, s_abs, head_dim: int, dtype: str, what: str = "",
                       rerotated_keys: bool = False, gamma: float = None, rounded_p_sum: bool = False):
    """Every element of o and lse within the error-model bars of ``decode_bars``.  Returns
    the largest ratio error / bar of each (<= 1 passes)."""
    bar_o, bar_lse = decode_bars(ref_o, ref_lse, a, s_abs, head_dim, dtype, rerotated_keys, gamma, rounded_p_sum)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    ro = np.abs(o - ref_o) / bar_o
    rl = np.abs(lse - ref_lse) / bar_lse
    worst_o, worst_l = float(ro.max()), float(rl.max())
    assert worst_o <= 1.0, (f"{what}: O error {float(np.abs(o - ref_o).flat[ro.argmax()]):.3g} exceeds its "
                            f"error-model bar {float(bar_o.flat[ro.argmax()]):.3g} (element {int(ro.argmax())})")
    assert worst_l <= 1.0, (f"{what}: LSE error {float(np.abs(lse - ref_lse).flat[rl.argmax()]):.3g} exceeds its "
                            f"error-model bar {float(bar_lse.flat[rl.argmax()]):.3g} (row {int(rl.argmax())})")
    return worst_o, worst_l


def plant_queries(sc: W.Scenario, rng, scale_up: float = 40.0, idx=None):
    """Queries that each single out one key: row (i, h) becomes scale_up * k_j / |k_j|^2
    (over sm_scale) for a key j of query i's visible context (KV head of h; drawn uniformly,
    or idx[i][h]), rounded to the storage type, so that row's softmax puts all but ~e^-20
    of its weight on key j and its output is v_j.  Returns (q in storage form [n, Hq, d],
    planted v [n, Hq, d] in fp64, planted context indices [n, Hq]).  Keys come from the
    oracle's page table."""
    from oracle import pagetable as pt
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    n, hq, d = len(sc.queries), sc.n_q_heads, sc.head_dim
    g = hq // sc.n_kv_heads
    q = np.zeros((n, hq, d))
    vp = np.zeros((n, hq, d))
    given = idx
    idx = np.zeros((n, hq), np.int64)
    for i, sid in enumerate(sc.queries):
        k, v = table.materialise(sid)
        for h in range(hq):
            j = int(rng.integers(0, k.shape[0])) if given is None else int(given[i][h])
            kj = k[j, h // g]
            q[i, h] = scale_up * kj / (float(kj @ kj) * sc.sm_scale)
            vp[i, h] = v[j, h // g]
            idx[i, h] = j
    qs = W.to_bf16_bits(q) if sc.dtype == "bf16" else q.astype(np.float32)
    return qs, vp, idx


def subscenario(sc: W.Scenario, seq_ids):
    """The operations of independent sequences `seq_ids` only (creation order kept), with
    sequence ids renumbered; used to run the oracle one request at a time."""
    remap = {}
    ops = []
    blocks = []
    nxt = 0
    owner = []
    for op in sc.ops:  # ids in creation order
        if op[0] in ("create", "fork"):
            owner.append(op)
    sid = 0
    keep_ops = []
    for op in sc.ops:
        if op[0] == "create":
            if sid in seq_ids:
                remap[sid] = nxt
                nxt += 1
                keep_ops.append(("create",))
            sid += 1
        elif op[0] == "fork":
            raise ValueError("subscenario is for independent sequences")
        elif op[1] in remap:
            if op[0] == "append":
                blocks.append(sc.blocks[op[2]])
                keep_ops.append(("append", remap[op[1]], len(blocks) - 1))
            else:
                keep_ops.append((op[0], remap[op[1]]) + tuple(op[2:]))
    qi = [sc.queries.index(s) for s in seq_ids]
    sub = W.Scenario(name=sc.name + "_sub", n_q_heads=sc.n_q_heads, n_kv_heads=sc.n_kv_heads, head_dim=sc.head_dim,
                     page_size=sc.page_size, dtype=sc.dtype, sm_scale=sc.sm_scale, rope_theta=sc.rope_theta,
                     n_pages=sc.n_pages, ops=keep_ops, blocks=blocks, queries=[remap[s] for s in seq_ids],
                     q=sc.q[qi])
    return sub


def check_close(got: np.ndarray, ref: np.ndarray, max_abs: float, mean_abs: float, what: str = ""):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mn = float(err.max()), float(err.mean())
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3g} (<= {max_abs}), mean-abs {mn:.3g} (<= {mean_abs})"
    return mx, mn


def check_decode_both(o, lse, ref, head_dim: int, dtype: str, what: str, rerotated_keys: bool = False,
                      gamma: float = None, rounded_p_sum: bool = False):
    """The coarse gate (bf16: max-abs 2e-2 / mean-abs 2e-3; fp32: 1e-4; LSE 2e-3) and the
    error-model bars, for outputs o [.., d] / lse against ref = (o, lse, a, s_abs) of the
    oracle with magnitudes.  Returns (max-abs, mean-abs, worst O / bar, worst LSE / bar)."""
    ro, rl, a, s_abs = ref
    tol = (2e-2, 2e-3) if dtype == "bf16" else (1e-4, 1e-4)
    mx, mn = check_close(o, ro, *tol, what)
    check_close(lse, rl, 2e-3, 2e-3, what + " lse")
    wo, wl = check_decode_model(o, lse, ro, rl, a, s_abs, head_dim, dtype, what, rerotated_keys, gamma,
                                rounded_p_sum)
    return mx, mn, wo, wl
