"""The decode error-model bars (tests/harness.py: decode_bars) have teeth at full size,
on the CPU: an oracle result over a context missing one page, or with one page's
contents replaced by another page's, is rejected by the bars derived for the true
context, although it passes the coarse max-abs 2e-2 / mean-abs 2e-3 / LSE 2e-3 gate.
Planted-key queries single out one key per row (closed form: O = v of that key)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as att, pagetable as pt
from tests.harness import check_decode_model, decode_bars, plant_queries


def _table(sc):
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    return table


def _rejected(o, lse, ref):
    try:
        check_decode_model(o, lse, *ref, head_dim=128, dtype="bf16")
    except AssertionError:
        return True
    return False


def _coarse_pass(o, lse, ro, rl):
    return np.abs(o - ro).max() <= 2e-2 and np.abs(o - ro).mean() <= 2e-3 and np.abs(lse - rl).max() <= 2e-3


@pytest.mark.parametrize("make,seq,pages", [
    (W.shared_prefix_fork, 1, (700, 2047, 2100)),   # two pages of the shared prefix, one private
    (W.octopus_dag, 1, (1500, 4200, 4700)),         # root, own private part, near the own end
])
def test_bars_reject_a_missing_or_foreign_page_at_full_size(make, seq, pages):
    sc = make()
    i = sc.queries.index(seq)
    q = W.storage_to_f64(sc.q, sc.dtype)[i:i + 1]
    table = _table(sc)
    ref = att.decode(table, [seq], q, sc.sm_scale, with_magnitudes=True)
    ro, rl = ref[0], ref[1]
    k, v = table.materialise(seq)  # own tokens, then mounts
    for L in pages:
        keep = np.ones(k.shape[0], bool)
        keep[16 * L:16 * L + 16] = False  # the same context without that page's 16 tokens
        o2, l2 = att.attend_heads(q[0], k[keep], v[keep], sc.sm_scale)
        o2, l2 = o2[None], l2[None]
        assert _coarse_pass(o2, l2, ro, rl), "the coarse gate was expected to be blind here"
        assert _rejected(o2, l2, ref), f"missing page {L} passed the error-model bars"
        k3, v3 = k.copy(), v.copy()  # a wrong page: another page's keys and values
        k3[16 * L:16 * L + 16] = k[16 * L + 48:16 * L + 64]
        v3[16 * L:16 * L + 16] = v[16 * L + 48:16 * L + 64]
        o3, l3 = att.attend_heads(q[0], k3, v3, sc.sm_scale)
        assert _rejected(o3[None], l3[None], ref), f"foreign contents in page {L} passed the error-model bars"
    # and the true result passes them, with room to spare for the kernel's rounding
    assert not _rejected(ro, rl, ref)


def test_bars_scale_with_the_terms():
    # the bar is linear in a and |O| and grows with the score magnitude
    a = np.full((1, 1, 4), 0.5)
    o = np.full((1, 1, 4), 0.1)
    b1, l1 = decode_bars(o, np.zeros((1, 1)), a, np.full((1, 1), 10.0), 128, "bf16")
    b2, l2 = decode_bars(o, np.zeros((1, 1)), 2 * a, np.full((1, 1), 10.0), 128, "bf16")
    b3, l3 = decode_bars(o, np.zeros((1, 1)), a, np.full((1, 1), 20.0), 128, "bf16")
    assert np.all(b2 > b1) and np.all(b3 > b1) and np.all(l3 > l1) and np.all(l2 == l1)
    assert np.allclose(b1, (2.0 ** -8 + np.expm1(2 * 130 * 2.0 ** -24 * 10) + 2.0 ** -15) * 0.5
                       + 2.0 ** -8 * 0.1 + 1e-7)


def test_planted_queries_single_out_their_key():
    # closed form: a row whose query is a large multiple of one key attends to that key only
    sc = W.fork_scenario(prefix=300, branches=3, private=[20, 0, 45], hq=8, hkv=2, d=128, seed=7)
    qs, vp, idx = plant_queries(sc, np.random.default_rng(0))
    o, lse = att.decode(_table(sc), sc.queries, W.storage_to_f64(qs, sc.dtype), sc.sm_scale)
    assert np.abs(o - vp).max() < 1e-6
    assert len(np.unique(idx)) > 10
