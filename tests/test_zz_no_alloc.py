"""fork_attn_decode_static (no workspace argument, library-held device array) against
fork_attn_decode with a caller workspace: bit-identical outputs on consecutive calls,
the second with a smaller input, then the first pool again (its plan re-uploaded after
another pool's call used the array); each also within the oracle's bars."""
import numpy as np
import pytest

import workloads as W
from tests.harness import build_device_pool, check_decode_both, oracle_decode, out_to_f64, to_torch

pytestmark = pytest.mark.gpu


def _both(sc, pool, label):
    import torch
    import fork_attention_decode_amd as fa
    print(f"[case] static-buffer decode vs workspace decode: {label}", flush=True)
    q = to_torch(sc.q, sc.dtype)
    o1, l1 = pool.decode(sc.queries, q, sc.sm_scale)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    fa.fork_attn_decode_static(pool.handle, sc.queries, sc.n_q_heads, q.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                               sc.sm_scale, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), label
    check_decode_both(out_to_f64(o2, sc.dtype), l2.double().cpu().numpy(), oracle_decode(sc, with_magnitudes=True),
                      sc.head_dim, sc.dtype, label)
    return o2, l2


def test_static_decode_equals_workspace_decode():
    import torch
    big = W.fork_scenario(prefix=3000, branches=6, private=[40, 0, 300, 17, 16, 1000], hq=16, hkv=4, d=128, seed=81)
    small = W.fork_scenario(prefix=200, branches=2, private=[5, 33], hq=8, hkv=2, d=128, seed=82)
    pb, _ = build_device_pool(big)
    ps, _ = build_device_pool(small)
    ob, lb = _both(big, pb, "first call")
    _both(small, ps, "second call, smaller input")
    ob2, lb2 = _both(big, pb, "the first pool again")
    assert torch.equal(ob, ob2) and torch.equal(lb, lb2)
    print("[ok] static-buffer decode", flush=True)
