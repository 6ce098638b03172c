"""Benchmark of the fork / DAG attention hot path on one MI355X.  Prints ONE JSON line.

Step (the headline `value`): one fork_attn_decode over every branch of the shared-prefix
fork workload -- 16 branches x 32 query heads, 8 KV heads, d = 128, bf16, a 32,768-token
shared prefix + 2,048 private tokens per branch, page 16 -- with every input resident
in HBM.  `value` = branch-tokens/s (branches decoded per second of wall clock over the
timed steps).  `roofline` prices the same step (decode_kernel from fork_attn_partials +
merge_kernel from fork_attn_merge) against MI355X's 8 TB/s HBM with its algorithmic
bytes (each unique KV byte once + Q read + O written), timed with HIP events on the
replaying stream; `roofline.kernel_only` prices the decode kernel alone.  `ceilings`
holds the achievable read rate and matrix-core rate measured by the library's probe
kernels.  Steps rotate over several identical pool copies so no step finds its KV in
the last-level cache left by the previous one.

Further objects in the same line (each timed the same way, on its own workload):
  prefill       the packed DAG prefill attention kernel (dag_attn_run) on the
                81,920-token packed workload, priced against 2.5 PFLOP/s dense bf16 with
                its algorithmic FLOPs (4 d per visible query-key pair per query head);
  octopus_dag   decode over the Octopus-style DAG (mounted sibling blocks);
  akv           drop + repos compaction of 16 x 131,072-token requests (40 % dropped),
                then decode over the compacted requests.
cpu_baseline times the fp64 oracle on a bounded sample of the headline workload, and in
full on the tiny fork workload; the Octopus leg times it over every thread and the AKV
leg over one request.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fork-decode branch-tokens/s + achieved HBM GB/s (% of peak); DAG-prefill % MFMA peak"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_traffic.json")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_kernel_traffic.json")
PREFILL_FLOPS = 27488461783040  # 4 * 128 * 1,677,762,560 visible pairs * 32 query heads
PREFILL_BWD_FLOPS = 68721154457600  # 10 * 128 * pairs * heads: S again, dP, dV, dK, dQ (2.5 x the forward)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_traffic():
    """HBM bytes per prefill_kernel launch (FETCH + WRITE) from the committed rocprofv3
    runs, or None once the kernel source differs from the profiled one."""
    import hashlib
    try:
        rec = json.load(open(PREFILL_TRAFFIC_FILE))
        h = hashlib.sha256()
        for f in rec["source_files"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["source_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def measured_traffic():
    """HBM bytes per decode step and per decode_kernel launch from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs ({"step": ..., "decode_kernel": ...}), or None
    once the kernel or planner sources differ from the profiled ones."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        h = hashlib.sha256()
        for f in rec["source_files"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return {"step": rec["traffic_bytes_per_step"], "decode_kernel": rec["traffic_bytes_per_decode_launch"]}
    except (OSError, KeyError, ValueError):
        return None


class DecodeBench:
    """fork_attn_partials + fork_attn_merge over prepared pools (plans cached)."""

    def __init__(self, pools, sc, q):
        import torch
        import fork_attention_decode_amd as fa
        self.fa, self.torch = fa, torch
        self.pools, self.sc, self.q = pools, sc, q
        self.n, self.hq, self.d = q.shape
        self.out = torch.empty_like(q)
        self.lse = torch.empty((self.n, self.hq), dtype=torch.float32, device=q.device)
        self.wss = []
        for p in pools:
            need = fa.fork_attn_workspace_size(p.handle, sc.queries, self.hq)
            self.wss.append(torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device))
        self.stream = torch.cuda.current_stream().cuda_stream
        self.stats = pools[0].plan_stats()
        es = 2 if sc.dtype == "bf16" else 4
        self.kernel_bytes = self.stats["unique_kv_bytes"] + q.numel() * es  # decode kernel: unique KV + Q
        self.step_bytes = self.kernel_bytes + q.numel() * es                # whole step: + O written

    def step(self, i, ev=None, stream=None, merge=True):
        p, ws = self.pools[i % len(self.pools)], self.wss[i % len(self.pools)]
        s = stream or self.stream
        if ev:
            ev[0].record()
        self.fa.fork_attn_partials(p.handle, self.sc.queries, self.hq, self.q.data_ptr(), self.sc.sm_scale,
                                   ws.data_ptr(), ws.numel(), s)
        if ev:
            ev[1].record()
        if merge:
            self.fa.fork_attn_merge(p.handle, self.sc.queries, self.hq, self.out.data_ptr(), self.lse.data_ptr(),
                                    ws.data_ptr(), ws.numel(), s)
        if ev:
            ev[2].record()

    def host_call_us(self, reps=20):
        """Host time of one fork_attn_partials call (ctypes call, plan lookup, launch) with
        the plan cached, and when the plan must be rebuilt and uploaded (the query list
        changes between calls).  Runs before the timed work; leaves the usual plan cached."""
        import numpy as np
        torch = self.torch
        p, ws = self.pools[0], self.wss[0]
        seqs, alt = list(self.sc.queries), list(reversed(self.sc.queries))

        def call(qs):
            t0 = time.perf_counter()
            self.fa.fork_attn_partials(p.handle, qs, self.hq, self.q.data_ptr(), self.sc.sm_scale, ws.data_ptr(),
                                       ws.numel(), self.stream)
            return (time.perf_counter() - t0) * 1e6

        call(seqs)
        torch.cuda.synchronize()
        cached = [call(seqs) for _ in range(reps)]
        torch.cuda.synchronize()
        rebuilt = []
        for i in range(reps):
            rebuilt.append(call(alt if i % 2 == 0 else seqs))
            torch.cuda.synchronize()
        call(seqs)
        torch.cuda.synchronize()
        return {"plan_cached_us_median": float(np.median(cached)), "plan_rebuilt_us_median": float(np.median(rebuilt)),
                "note": "host wall time of one fork_attn_partials call from Python (ctypes included); rebuilt = the "
                        "query list changed, so the segment plan is recomputed and uploaded"}

    def capture(self, steps, merge=True):
        """A HIP graph of `steps` decode steps (pools rotated as in the eager loop), or with
        merge=False of `steps` back-to-back decode kernels.  The plans are cached by then, so
        each call is a bare kernel launch and the graph replays exactly the eager work."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            s = torch.cuda.current_stream().cuda_stream
            for i in range(steps):
                self.step(i, stream=s, merge=merge)
        torch.cuda.synchronize()
        return g

    def run_graph(self, steps):  # -> wall s of `steps` graph-replayed steps, step us (events), decode-kernel us
        """The step loop as one graph replay (no per-launch host work), bracketed by the
        host clock and by HIP events on the replaying stream; then the decode kernel's
        launch duration: HIP events around a replay of `steps` back-to-back decode kernels,
        divided by `steps` (ROCm cannot record timing events inside a graph)."""
        torch = self.torch
        g = self.capture(steps)
        g.replay()
        torch.cuda.synchronize()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ea.record()
        g.replay()
        eb.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_us = ea.elapsed_time(eb) * 1e3 / steps
        gd = self.capture(steps, merge=False)
        gd.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        gd.replay()
        b.record()
        torch.cuda.synchronize()
        del g, gd
        return wall, step_us, a.elapsed_time(b) * 1e3 / steps

    def settle(self, seconds):
        """Untimed steps for `seconds` of wall clock before the warmup: the first few
        hundred launches of a fresh process run several times slower than the steady state
        (measured: ~200 us per step for the first ~200 steps, then ~52 us), whatever the
        warmup count asked for."""
        torch = self.torch
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < seconds:
            self.step(i)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return i

    def run(self, steps, warmup, settle_s=0.0):  # -> wall seconds, decode-kernel ms, step ms
        import numpy as np
        torch = self.torch
        self.settled_steps = self.settle(settle_s) if settle_s > 0 else 0
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, ev[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        k_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
        s_ms = np.array([a.elapsed_time(c) for a, _, c in ev])
        return wall, k_ms, s_ms

    def summary(self, steps, warmup, settle_s=0.5):
        import numpy as np
        wall, k_ms, s_ms = self.run(steps, warmup, settle_s)
        t_k = float(np.mean(k_ms)) * 1e-3
        t_s = float(np.mean(s_ms)) * 1e-3
        return {
            "branch_tokens_per_s": self.n / (wall / steps),
            "ms_per_step_wall": wall * 1e3 / steps,
            "decode_kernel_us_mean": t_k * 1e6,
            "decode_kernel_GBps": self.kernel_bytes / t_k / 1e9,
            "decode_kernel_frac_of_8TBps": self.kernel_bytes / t_k / 1e9 / HBM_PEAK_GBPS,
            "step_us_mean_events": t_s * 1e6,
            "step_GBps": self.step_bytes / t_s / 1e9,
            "step_frac_of_8TBps": self.step_bytes / t_s / 1e9 / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": self.kernel_bytes,
            "steps": steps,
            "settle_steps": self.settled_steps,
            "plan": self.stats,
        }


def bench_prefill(reps, warmup, cpu_budget=0.0):
    """dag_attn_run (attention kernel alone, HIP events on its stream) on the packed DAG
    workload; the preparation (K / V relayout, column packing, row order) is timed apart.
    With cpu_budget > 0 the fp64 oracle is also timed on query rows drawn uniformly at
    random for about that many seconds, and its full-workload time extrapolated (mean time
    per row x T)."""
    import numpy as np
    import torch
    import workloads as W
    import fork_attention_decode_amd as fa
    from tests.harness import to_torch
    log("prefill: generating the packed DAG workload")
    pi = W.dag_prefill()
    mask = fa.DagMask(pi.segments, pi.edges, pi.T, pi.block)
    q, k, v = (to_torch(x, "bf16") for x in (pi.q, pi.k, pi.v))
    host = (pi.q, pi.k, pi.v) if cpu_budget > 0 else None
    pi.q = pi.k = pi.v = None
    hq, hkv = q.shape[1], k.shape[1]
    out = torch.empty_like(q)
    lse = torch.empty((hq, pi.T), dtype=torch.float32, device=q.device)
    ws = torch.empty(fa.dag_attn_workspace_size(pi.T, hq, hkv, 64, mask.nnz), dtype=torch.uint8, device=q.device)
    st = torch.cuda.current_stream().cuda_stream

    def prepare():
        fa.dag_attn_prepare(k.data_ptr(), v.data_ptr(), pi.T, hq, hkv, 128, mask.row_ptr.data_ptr(),
                            mask.col.data_ptr(), mask.kind.data_ptr(), mask.nnz, 64, ws.data_ptr(), ws.numel(), st)

    def run():
        fa.dag_attn_run(q.data_ptr(), out.data_ptr(), lse.data_ptr(), pi.T, hq, hkv, 128, mask.row_ptr.data_ptr(),
                        mask.nnz, 64, pi.sm_scale, ws.data_ptr(), ws.numel(), st)

    prepare()
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    log(f"prefill: timing {reps} calls")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        prepare()
        e[1].record()
        run()
        e[2].record()
    torch.cuda.synchronize()
    prep_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    run_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    t = float(np.mean(run_ms)) * 1e-3
    tflops = PREFILL_FLOPS / t / 1e12
    cpu = None
    if host is not None:
        cpu = prefill_cpu_baseline(pi, host, cpu_budget)
    out_obj = {
        "workload": "packed_dag_prefill (16,384-token prefix + 8 x 8,192 branches, 12 edges of 2,048 tokens; "
                    "T = 81,920; 32 / 8 heads, d = 128, bf16)",
        "block_pairs": mask.nnz,
        "visible_token_pairs": 1677762560,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_PEAK_TFLOPS, "traffic": prefill_traffic(),
                     "kernel": "prefill_kernel (dag_attn_run)", "algorithmic_flops_per_launch": PREFILL_FLOPS,
                     "kernel_ms_mean": t * 1e3, "kernel_ms_p10": float(np.percentile(run_ms, 10)),
                     "kernel_ms_p90": float(np.percentile(run_ms, 90))},
        "prepare_ms_mean": float(np.mean(prep_ms)),
        "call_ms_mean": float(np.mean(prep_ms + run_ms)),
        "reps": reps,
    }
    if cpu is not None:
        out_obj["cpu_baseline"] = cpu
    return out_obj


def bench_prefill_bwd(reps, warmup):
    """dag_attn_backward (the whole call: operand images, mask transpose, dK / dV and dQ
    passes; HIP events on its stream) on the packed DAG workload, after one forward for
    out and lse; the upstream gradient is a seeded N(0, 1) draw in bf16."""
    import numpy as np
    import torch
    import workloads as W
    import fork_attention_decode_amd as fa
    from tests.harness import to_torch
    log("prefill backward: generating the packed DAG workload")
    pi = W.dag_prefill()
    mask = fa.DagMask(pi.segments, pi.edges, pi.T, pi.block)
    q, k, v = (to_torch(x, "bf16") for x in (pi.q, pi.k, pi.v))
    do = to_torch(W.to_bf16_bits(np.random.default_rng(67).standard_normal((pi.T, 32, 128))), "bf16")
    pi.q = pi.k = pi.v = None
    out, lse = fa.prefill(q, k, v, mask, pi.sm_scale)
    hq, hkv = q.shape[1], k.shape[1]
    dq = torch.empty((pi.T, hq, 128), dtype=torch.float32, device=q.device)
    dk = torch.empty((pi.T, hkv, 128), dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    ws = torch.empty(fa.dag_attn_backward_workspace_size(pi.T, hq, hkv, 64, mask.nnz), dtype=torch.uint8,
                     device=q.device)
    st = torch.cuda.current_stream().cuda_stream

    def run():
        fa.dag_attn_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), do.data_ptr(), lse.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), pi.T, hq, hkv, 128,
                             mask.row_ptr.data_ptr(), mask.col.data_ptr(), mask.kind.data_ptr(), mask.nnz, 64,
                             pi.sm_scale, ws.data_ptr(), ws.numel(), st)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    log(f"prefill backward: timing {reps} calls")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        run()
        e[1].record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    t = float(np.mean(ms)) * 1e-3
    tflops = PREFILL_BWD_FLOPS / t / 1e12
    return {
        "workload": "packed_dag_prefill backward (same mask and shapes as the forward; dq fp32 [T][32][128], "
                    "dk / dv fp32 [T][8][128])",
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "dag_attn_backward (whole call)", "algorithmic_flops_per_call": PREFILL_BWD_FLOPS,
                     "call_ms_mean": t * 1e3, "call_ms_p10": float(np.percentile(ms, 10)),
                     "call_ms_p90": float(np.percentile(ms, 90))},
        "note": "algorithmic FLOPs = 10 x 128 per visible (query, key) pair per query head (S recomputed, dP, dV, "
                "dK, dQ); the dQ pass recomputes S and dP once more, so the matrix cores execute 14 x 128",
        "reps": reps,
    }


def bench_window(n_steps=16, replays=20):
    """Steady-state decode on the shared-prefix workload: a window of n_steps steps (each
    appends one token to all 16 branches and decodes them) captured once in a HIP graph and
    replayed; HIP events around the replays.  A replay rewrites the same reserved slots
    with the same rows, so every replay does the window's full work."""
    import numpy as np
    import torch
    import workloads as W
    from tests.harness import build_device_pool, to_torch
    sc = W.shared_prefix_fork()
    sc.n_pages += 64
    log("window: building the shared-prefix pool")
    pool, _ = build_device_pool(sc)
    seqs = list(sc.queries)
    n, hq, hkv, d = len(seqs), sc.n_q_heads, sc.n_kv_heads, sc.head_dim
    rng = np.random.default_rng(81)
    kt = [to_torch(W.to_bf16_bits(rng.standard_normal((n, hkv, d)) / np.sqrt(d)), "bf16") for _ in range(n_steps)]
    vt = [to_torch(W.to_bf16_bits(rng.standard_normal((n, hkv, d))), "bf16") for _ in range(n_steps)]
    qt = [to_torch(W.to_bf16_bits(rng.standard_normal((n, hq, d))), "bf16") for _ in range(n_steps)]
    out = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((n, hq), dtype=torch.float32, device="cuda")
    t0 = time.perf_counter()
    ws = pool.window(seqs, hq, n_steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for st in range(n_steps):
            pool.window_step(st, kt[st], vt[st], qt[st], sc.sm_scale, out, lse)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(replays):
        g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    us_step = ev[0].elapsed_time(ev[1]) * 1e3 / (replays * n_steps)
    del ws, g
    # the same steps without a window: kv_append_batch then fork_attn_decode, eager; after
    # the first step the decode plan is patched (no replanning) -- host time of each call
    import fork_attention_decode_amd as fa
    st = torch.cuda.current_stream().cuda_stream
    wsd = torch.empty(fa.fork_attn_workspace_size(pool.handle, seqs, hq) + (1 << 20), dtype=torch.uint8,
                      device="cuda")
    app_us, dec_us = [], []
    for step in range(n_steps):
        h0 = time.perf_counter()
        pool.append_batch(seqs, kt[step], vt[step])
        h1 = time.perf_counter()
        fa.fork_attn_decode(pool.handle, seqs, hq, qt[step].data_ptr(), out.data_ptr(), lse.data_ptr(), sc.sm_scale,
                            wsd.data_ptr(), wsd.numel(), st)
        h2 = time.perf_counter()
        app_us.append((h1 - h0) * 1e6)
        dec_us.append((h2 - h1) * 1e6)
    torch.cuda.synchronize()
    patched = pool.plan_stats()["patched_changes"]
    # each unique KV byte once per step (the shared prefix once, each branch's own tokens
    # once, the window's new tokens included), averaged over the window's steps
    ctx_tokens = 32768 + n * 2048 + n * (n_steps + 1) / 2
    step_bytes = ctx_tokens * hkv * d * 2 * 2
    return {
        "algorithmic_bytes_per_step": step_bytes,
        "step_GBps": step_bytes / (us_step * 1e-6) / 1e9,
        "step_frac_of_8TBps": step_bytes / (us_step * 1e-6) / 8e12,
        "workload": "shared_prefix_fork_decode steady state (16 branches, 32,768-token prefix + 2,048 private each; "
                    "every step appends one token per branch, then decodes all 16)",
        "steps_per_window": n_steps,
        "us_per_step": us_step,
        "branch_tokens_per_s": n / (us_step * 1e-6),
        "host_plan_upload_ms_per_window": (t1 - t0) * 1e3,
        "host_capture_ms_per_window": (t2 - t1) * 1e3,
        "eager_steps": {"append_batch_host_us_median": float(np.median(app_us[1:])),
                        "decode_host_us_median": float(np.median(dec_us[1:])),
                        "decode_host_us_first": dec_us[0], "plan_patches": patched,
                        "note": "kv_append_batch + fork_attn_decode per step without a window, host wall time of each "
                                "call from Python (ctypes included); the first decode replans, later ones patch the "
                                "cached plan"},
        "timed": "HIP events around back-to-back replays of the captured window (page write + decode + merge per "
                 "step)",
    }


def bench_restore(reps=20, n_seg=4, seg_len=128):
    """Restore of n_seg segments of seg_len tokens (own positions) into one branch of the
    shared-prefix workload: kv_append per segment, then kv_causal_attend over the restored
    tokens (HIP events around kv_causal_attend on its stream)."""
    import numpy as np
    import torch
    import workloads as W
    import fork_attention_decode_amd as fa
    from tests.harness import build_device_pool, to_torch
    sc = W.shared_prefix_fork()
    sc.n_pages += 64
    log("restore: building the shared-prefix pool")
    pool, _ = build_device_pool(sc)
    seq, hq, hkv, d = sc.queries[0], sc.n_q_heads, sc.n_kv_heads, sc.head_dim
    rng = np.random.default_rng(83)
    for i in range(n_seg):
        k = to_torch(W.to_bf16_bits(rng.standard_normal((seg_len, hkv, d)) / np.sqrt(d)), "bf16")
        v = to_torch(W.to_bf16_bits(rng.standard_normal((seg_len, hkv, d))), "bf16")
        pool.append(seq, k=k, v=v, positions=np.arange(100000 * (i + 1), 100000 * (i + 1) + seg_len))
    n = n_seg * seg_len
    q = to_torch(W.to_bf16_bits(rng.standard_normal((n, hq, d))), "bf16")
    t0 = time.perf_counter()
    need = fa.kv_causal_attend_workspace_size(pool.handle, seq, n, hq)  # plans (cached for the calls below)
    host_plan_ms = (time.perf_counter() - t0) * 1e3
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((n, hq), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def run():
        fa.kv_causal_attend(pool.handle, seq, n, hq, q.data_ptr(), out.data_ptr(), lse.data_ptr(), sc.sm_scale,
                            ws.data_ptr(), ws.numel(), st)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        run()
        e[1].record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    ctx = int(pool.info(seq)[0])
    kv_bytes = ctx * hkv * d * 2 * 2
    # 4 d FLOPs per visible (restored token, key) pair per query head; token j sees ctx - n + j + 1 keys
    flops = 4 * d * hq * sum(ctx - n + j + 1 for j in range(n))
    tflops = flops / (float(np.mean(ms)) * 1e-3) / 1e12
    return {
        "workload": f"restore {n_seg} segments x {seg_len} tokens (own positions) into a branch of the shared-prefix "
                    f"workload, then causal attention of the {n} restored tokens over the {ctx}-token context",
        "us_mean": float(np.mean(ms)) * 1e3, "us_p10": float(np.percentile(ms, 10)) * 1e3,
        "host_plan_ms": host_plan_ms,
        "context_kv_bytes": kv_bytes,
        "rows": n * hq,
        "roofline": {"bound": "mfma", "unit": "TFLOP/s", "peak": 2500.0, "algorithmic_flops_per_call": flops,
                     "achieved": tflops, "frac": tflops / 2500.0},
        "note": "the attention runs as a split-K tiled prefill: every workgroup takes 64 restored tokens x 4 query "
                "heads of one KV head over one piece of the key range (32 x 32 x 16 matrix instructions), copying the "
                "context's K and V straight from the pool's pages into its LDS ring (the visible keys fill whole "
                "pages), and the pieces' partials are merged by log-sum-exp; the plan (host) is built once and "
                "cached, the events enclose the kernels",
    }


def bench_select(reps, warmup):
    """Key scoring + keep selection (AgentKV's choice of entries before a compression) on
    one 131,072-token sequence (32 / 8 heads, d = 128, bf16) with 32 representative
    queries: kv_score and kv_select_keep timed with HIP events on their stream, then one
    score -> select -> drop (no repos) end to end on the host clock."""
    import numpy as np
    import torch
    import fork_attention_decode_amd as fa
    import workloads as W
    from tests.harness import build_device_pool, to_torch
    n_ctx, n_rep = 131072, 32
    log("select: building a 131,072-token sequence")
    sc = W.drop_scenario(requests=1, ctx=n_ctx, frac=0.0, hq=32, hkv=8, d=128, seed=3, repos=False)
    pool, _ = build_device_pool(sc)
    seq = 0
    n_tok = pool.info(seq)[0]
    qb = W.to_bf16_bits(np.random.default_rng(50).standard_normal((n_rep, 32, 128)))
    q_rep = to_torch(qb, "bf16")
    ws = torch.empty(fa.kv_score_workspace_size(pool.handle, seq, n_rep, 32), dtype=torch.uint8, device="cuda")
    scores = torch.empty(n_tok, dtype=torch.float32, device="cuda")
    keep = torch.empty(n_tok, dtype=torch.uint8, device="cuda")
    sel_ws = torch.empty(fa.kv_select_workspace_size(n_tok), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    budget = int(0.6 * n_tok)

    def score():
        fa.kv_score(pool.handle, seq, q_rep.data_ptr(), n_rep, 32, sc.sm_scale, scores.data_ptr(), ws.data_ptr(),
                    ws.numel(), st)

    def select():
        fa.kv_select_keep(scores.data_ptr(), n_tok, budget, keep.data_ptr(), sel_ws.data_ptr(), sel_ws.numel(), st)

    for _ in range(warmup):
        score()
        select()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        score()
        e[1].record()
        select()
        e[2].record()
    torch.cuda.synchronize()
    sc_us = np.array([a.elapsed_time(b) for a, b, _ in ev]) * 1e3
    se_us = np.array([b.elapsed_time(c) for _, b, c in ev]) * 1e3
    k_bytes = n_tok * 8 * 128 * 2
    alg = 2 * k_bytes  # every key's logits twice: normalisers, then scores
    t0 = time.perf_counter()
    mask = pool.select_and_drop(seq, q_rep, sc.sm_scale, budget, repos=False)
    torch.cuda.synchronize()
    e2e_ms = (time.perf_counter() - t0) * 1e3
    return {
        "workload": "agentkv_select (one 131,072-token sequence, 32 / 8 heads, d = 128, bf16; 32 representative "
                    "queries; keep 60 %)",
        "score_us_mean": float(np.mean(sc_us)), "score_us_p10": float(np.percentile(sc_us, 10)),
        "score_us_p90": float(np.percentile(sc_us, 90)),
        "algorithmic_bytes": alg,
        "score_GBps": alg / (float(np.mean(sc_us)) * 1e-6) / 1e9,
        "score_frac_of_8TBps": alg / (float(np.mean(sc_us)) * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "note": "algorithmic bytes = the sequence's K read twice (normaliser pass, then score pass); the events "
                "enclose the whole kv_score call (its chunk list is uploaded by the first call only)",
        "select_us_mean": float(np.mean(se_us)),
        "select_drop_end_to_end_ms": e2e_ms, "kept": int(mask.sum()), "reps": reps,
    }


def bench_octopus(steps, warmup, cpu_timing=False):
    """Decode over the Octopus-style DAG: eager steps with per-launch events, then the
    timed steps as one graph replay (as the headline), two pool copies rotated (each
    537 MB of KV, beyond the last-level cache).  cpu_timing: the fp64 oracle over every
    thread of the same workload, timed once."""
    import workloads as W
    from tests.harness import build_device_pool, to_torch
    log("octopus_dag: building 2 pool copies")
    sc = W.octopus_dag()
    pools = [build_device_pool(sc)[0] for _ in range(2)]
    db = DecodeBench(pools, sc, to_torch(sc.q, sc.dtype))
    d = db.summary(steps, warmup)
    wall, step_us, k_us = db.run_graph(steps)
    d["graph"] = {"branch_tokens_per_s": db.n / (wall / steps), "us_per_step_wall": wall * 1e6 / steps,
                  "step_us_events": step_us, "decode_kernel_us": k_us,
                  "step_GBps": db.step_bytes / (step_us * 1e-6) / 1e9,
                  "step_frac_of_8TBps": db.step_bytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                  "decode_kernel_frac_of_8TBps": db.kernel_bytes / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                  "step_algorithmic_bytes": db.step_bytes}
    d["branch_tokens_per_s"] = d["graph"]["branch_tokens_per_s"]
    d["timed"] = "graph replay of the timed steps (as the headline); eager per-launch events in the other fields"
    d["workload"] = ("octopus_dag_decode (65,536-token root, 8 threads x 8,192 private tokens, each mounting "
                     "the last 4,096 tokens of 2 siblings)")
    del db, pools
    if cpu_timing:
        d["oracle_full"] = oracle_full_timing(sc, "every thread of the Octopus DAG workload")
    return d


def oracle_full_timing(sc, what):
    """The fp64 oracle over every query of a scenario once: page-table replay, then the
    materialising decode of each query (timed apart)."""
    import workloads as W
    from oracle import attention as att, pagetable as pt
    t0 = time.perf_counter()
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    t1 = time.perf_counter()
    q = W.storage_to_f64(sc.q, sc.dtype)
    att.decode(table, sc.queries, q, sc.sm_scale)
    t2 = time.perf_counter()
    return {"kind": "oracle", "what": what, "queries": len(sc.queries), "decode_s": t2 - t1, "replay_s": t1 - t0,
            "branch_tokens_per_s": len(sc.queries) / (t2 - t1), "cores": len(os.sched_getaffinity(0))}


def measure_ceilings():
    """Achievable ceilings on this GPU, by the library's probe kernels: a streaming read of
    2 GiB and of 268,435,456 B (the shared-prefix decode's KV, in one launch), and a
    register-only bf16 matrix-core loop (clock implied at 4,096 FLOP / clock / CU)."""
    import numpy as np
    import torch
    import fork_attention_decode_amd as fa
    st = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    out = {}
    for label, nbytes in (("read_2GiB", 2 << 30), ("read_268MB", 268435456)):
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2 if nbytes < (1 << 30) else 1)]
        for b in bufs:
            b.fill_(1)
        for b in bufs:
            fa.kv_probe_stream_read(b.data_ptr(), nbytes, sink.data_ptr(), st)
        ms = []
        for i in range(10):
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fa.kv_probe_stream_read(bufs[i % len(bufs)].data_ptr(), nbytes, sink.data_ptr(), st)
            e.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(e))
        out[label] = {"GBps": nbytes / (float(np.median(ms)) * 1e-3) / 1e9, "us_median": float(np.median(ms)) * 1e3}
        del bufs
    # device-to-device copy of 1 GiB (torch's copy kernel): read + write traffic ceiling
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(3)
    dst.copy_(src)
    ms = []
    for _ in range(5):
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(e))
    out["copy_1GiB"] = {"GBps_read_plus_write": 2 * (1 << 30) / (float(np.median(ms)) * 1e-3) / 1e9,
                        "us_median": float(np.median(ms)) * 1e3}
    del src, dst
    n_iter, n_wg = 2000, 2048
    flops = 4 * 8 * n_iter * 32768 * n_wg
    fa.kv_probe_mfma_loop(200, n_wg, sink.data_ptr(), st)
    ms = []
    for _ in range(5):
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fa.kv_probe_mfma_loop(n_iter, n_wg, sink.data_ptr(), st)
        e.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(e))
    tf = flops / (float(np.median(ms)) * 1e-3) / 1e12
    out["mfma_bf16"] = {"TFLOPs": tf, "implied_clock_GHz": tf * 1e12 / (256 * 4096) / 1e9,
                        "us_median": float(np.median(ms)) * 1e3}
    out["note"] = ("probe kernels of the library (kv_probe_stream_read, kv_probe_mfma_loop) and torch's device copy, "
                   "HIP events, median of 10 / 5 launches; the vendor peaks are 8,000 GB/s and 2,500 TFLOP/s")
    return out


def bench_akv(steps, warmup, cpu_timing=False):
    """Drop + repos of every request in one kv_drop_batch call (its plan upload and
    compaction launch timed with HIP events behind a device sleep that covers the host
    planning), then decode over the compacted pool."""
    import numpy as np
    import torch
    import workloads as W
    import fork_attention_decode_amd as fa
    from tests.harness import to_torch
    log("akv: generating 16 x 131,072-token requests")
    sc = W.akv_drop_repos()
    pool = fa.Pool(sc.n_kv_heads, sc.head_dim, sc.n_pages, dtype=sc.dtype, rope_theta=sc.rope_theta)
    drops, tail, dropped = [], [], set()
    for op in sc.ops:
        if op[0] == "create":
            pool.seq_create()
        elif op[0] == "drop":
            drops.append(op)
            dropped.add(op[1])
        elif op[0] == "append" and op[1] not in dropped:
            blk = sc.blocks[op[2]]
            pool.append(op[1], to_torch(blk.k, sc.dtype), to_torch(blk.v, sc.dtype), positions=blk.pos)
            torch.cuda.synchronize()
        else:
            tail.append(op)
    moved = 0  # tokens the compaction rewrites: every slot from the first changed page on
    for _, sid, spans, _ in drops:
        gone = np.zeros(int(pool.info(sid)[0]), bool)
        for b, L in spans:
            gone[b:b + L] = True
        kept = np.nonzero(~gone)[0]
        diff = kept != np.arange(len(kept))
        first = int(np.argmax(diff)) if diff.any() else len(kept)
        moved += len(kept) - 16 * (first // 16)
    log("akv: compaction")
    # Each drop's device work (plan upload + compaction kernel) is bracketed by events on
    # the stream; a device sleep longer than the host planning sits before the first
    # event, so the window holds no host time.  The sleep is calibrated first.
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    torch.cuda._sleep(50_000_000)
    c1.record()
    torch.cuda.synchronize()
    cycles_per_ms = 50_000_000 / max(c0.elapsed_time(c1), 1e-3)
    # all 16 drops in one kv_drop_batch call: one plan upload, one compaction launch
    assert all(op[3] for op in drops)
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(cycles_per_ms * 400))  # 400 ms of device time
    ea.record()
    t0 = time.perf_counter()
    pool.drop_batch([op[1] for op in drops], [op[2] for op in drops], repos=True)
    host_s = time.perf_counter() - t0
    eb.record()
    torch.cuda.synchronize()
    comp_ms = ea.elapsed_time(eb)
    covered = host_s < 0.38
    dev_ms = [comp_ms]
    assert pool.sync_status() == 0
    for op in tail:
        blk = sc.blocks[op[2]]
        pool.append(op[1], to_torch(blk.k, sc.dtype), to_torch(blk.v, sc.dtype), positions=blk.pos)
    torch.cuda.synchronize()
    comp_bytes = moved * 4 * sc.n_kv_heads * sc.head_dim * 2  # read + write of K and V
    d = DecodeBench([pool], sc, to_torch(sc.q, sc.dtype)).summary(steps, warmup)
    d.update({"workload": "akv_drop_repos (16 x 131,072 tokens, 40 % dropped as 2,048-8,192-token spans, repos, "
                          "then 1 decode token each)",
              "compaction": {"device_ms_total": comp_ms, "moved_tokens": moved, "call": "kv_drop_batch (16 drops)",
                             "algorithmic_bytes": comp_bytes, "GBps": comp_bytes / (comp_ms * 1e-3) / 1e9,
                             "frac_of_8TBps": comp_bytes / (comp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                             "host_planning_ms_total": host_s * 1e3, "host_hidden_behind_device": covered,
                             "timed": "plan upload + compaction kernel of the one call, HIP events"},
              "note": "one pool, no rotation: its 5.15 GB of KV exceed the last-level cache"})
    if cpu_timing:
        from tests.harness import subscenario
        d["oracle_one_request"] = oracle_full_timing(subscenario(sc, [0]),
                                                     "one request (drop + repos replayed, then its decode)")
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup steps (launch path settling)")
    ap.add_argument("--copies", type=int, default=4, help="pool copies rotated between steps")
    ap.add_argument("--workload", default="shared_prefix_fork_decode",
                    choices=["shared_prefix_fork_decode", "octopus_dag_decode", "tiny_fork_decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work to sample")
    ap.add_argument("--only-decode", action="store_true", help="skip the prefill / DAG / AKV objects")
    ap.add_argument("--only-prefill", action="store_true", help="time the prefill object alone (profiling)")
    ap.add_argument("--only-akv", action="store_true", help="time the drop + repos object alone (profiling)")
    ap.add_argument("--only-select", action="store_true", help="time the key scoring object alone (profiling)")
    ap.add_argument("--only-prefill-bwd", action="store_true", help="time the prefill backward alone (profiling)")
    ap.add_argument("--only-window", action="store_true", help="time the steady-state decode window alone")
    ap.add_argument("--only-restore", action="store_true", help="time the segment restore alone")
    ap.add_argument("--only-octopus", action="store_true", help="time the Octopus DAG decode alone (profiling)")
    ap.add_argument("--prefill-reps", type=int, default=10)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, copy 256 MiB device to device once (a kernel of known "
                         "traffic to scale hardware byte counters against)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the library runs on one "
              f"MI355X; decode would shard by KV head with no exchange across GPUs).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    from tests.harness import build_device_pool, to_torch

    torch.cuda.set_device(0)

    def calibration():  # a device-to-device copy of 256 MiB: scales hardware byte counters
        if args.copy_calibration:
            src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()

    single = [(args.only_prefill, "prefill", lambda: bench_prefill(args.prefill_reps, 3)),
              (args.only_akv, "akv", lambda: bench_akv(max(20, args.steps // 4), 5)),
              (args.only_select, "agentkv_select", lambda: bench_select(20, 3)),
              (args.only_restore, "restore", lambda: bench_restore()),
              (args.only_window, "decode_window", lambda: bench_window()),
              (args.only_prefill_bwd, "prefill_backward", lambda: bench_prefill_bwd(5, 1)),
              (args.only_octopus, "octopus_dag", lambda: bench_octopus(max(20, args.steps // 4), 5))]
    for on, key, fn in single:
        if on:
            res = fn()
            calibration()
            print(json.dumps({key: res}))
            return
    sc = W.WORKLOADS[args.workload]()
    log(f"workload {args.workload}: building {args.copies} pool copies")
    pools = [build_device_pool(sc)[0] for _ in range(args.copies)]
    q = to_torch(sc.q, sc.dtype)
    db = DecodeBench(pools, sc, q)
    host_call = db.host_call_us()
    log(f"eager pass: {args.steps} steps after {args.warmup} warmup steps (per-launch events)")
    wall_eager, k_ms, s_ms = db.run(args.steps, args.warmup, args.settle)
    launch = "hip_graph"
    try:
        log(f"timed region: {args.steps} steps as one HIP graph replay")
        wall, step_us, k_us = db.run_graph(args.steps)
    except RuntimeError as e:  # no graph capture here: the eager loop is the timed region
        log(f"graph capture unavailable ({e}); timing the eager loop")
        launch, wall, k_us = "eager", wall_eager, float(np.mean(k_ms)) * 1e3
        step_us = float(np.mean(s_ms)) * 1e3
    calibration()
    ms_step = wall * 1e3 / args.steps
    t_kernel = k_us * 1e-6
    achieved = db.kernel_bytes / t_kernel / 1e9
    step_achieved = db.step_bytes / (step_us * 1e-6) / 1e9
    traffic = measured_traffic() if args.workload == "shared_prefix_fork_decode" else None
    ceilings = measure_ceilings() if not args.only_decode else None
    n_br, hq, d = q.shape
    result = {
        "metric": METRIC,
        "value": n_br / (ms_step * 1e-3),
        "unit": "branch-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sc.dtype,
        "data": "synthetic (seeded N(0,1) Q/V, K/sqrt(d), RoPE theta 1e6 pre-applied; no weights)",
        "config": {"workload": args.workload, "branches": n_br, "q_heads": hq, "kv_heads": sc.n_kv_heads,
                   "head_dim": d, "page_size": sc.page_size, "pool_copies_rotated": args.copies,
                   "settle_s": args.settle, "settle_steps": db.settled_steps, "launch": launch},
        "roofline": {"bound": "hbm", "achieved": step_achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": step_achieved / HBM_PEAK_GBPS,
                     "traffic": traffic["step"] if traffic else None,
                     "kernel": "decode step = decode_kernel (fork_attn_partials) + merge_kernel (fork_attn_merge)",
                     "algorithmic_bytes_per_step": db.step_bytes,
                     "algorithmic_bytes_note": "unique KV (each shared page once) + Q read + O written",
                     "step_us_mean": step_us,
                     "timing": ("HIP events around the graph replay of the timed steps" if launch == "hip_graph"
                                else "HIP events around each eager step"),
                     "frac_of_measured_read_ceiling": (step_achieved / ceilings["read_268MB"]["GBps"]
                                                       if ceilings else None),
                     "kernel_only": {"kernel": "decode_kernel (fork_attn_partials)",
                                     "algorithmic_bytes_per_launch": db.kernel_bytes,
                                     "achieved": achieved, "frac": achieved / HBM_PEAK_GBPS,
                                     "traffic": traffic["decode_kernel"] if traffic else None,
                                     "kernel_us_mean": t_kernel * 1e6,
                                     "kernel_timing": ("HIP events around a graph replay of back-to-back launches"
                                                       if launch == "hip_graph" else "HIP events around each launch"),
                                     "kernel_us_eager_events_mean": float(np.mean(k_ms)) * 1e3,
                                     "kernel_us_eager_events_p10": float(np.percentile(k_ms, 10)) * 1e3,
                                     "kernel_us_eager_events_p90": float(np.percentile(k_ms, 90)) * 1e3}},
        "ceilings": ceilings,
        "step": {"us_per_step_timed": ms_step * 1e3, "us_per_step_eager_wall": wall_eager * 1e6 / args.steps,
                 "achieved_GBps_timed": db.step_bytes / (ms_step * 1e-3) / 1e9,
                 "frac_of_peak_timed": db.step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                 "host_call": host_call,
                 "us_mean_events": float(np.mean(s_ms)) * 1e3, "algorithmic_bytes": db.step_bytes,
                 "achieved_GBps": db.step_bytes / (float(np.mean(s_ms)) * 1e-3) / 1e9,
                 "frac_of_peak": db.step_bytes / (float(np.mean(s_ms)) * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                 "merge_us_mean": float(np.mean(s_ms - k_ms)) * 1e3},
        "plan": db.stats,
    }
    del db, pools
    torch.cuda.empty_cache()

    if not args.only_decode:
        result["prefill"] = bench_prefill(args.prefill_reps, 3, 0.0 if args.no_cpu_baseline else 8.0)
        torch.cuda.empty_cache()
        result["decode_window"] = bench_window()
        torch.cuda.empty_cache()
        result["restore"] = bench_restore()
        torch.cuda.empty_cache()
        result["prefill_backward"] = bench_prefill_bwd(5, 1)
        torch.cuda.empty_cache()
        result["octopus_dag"] = bench_octopus(max(20, args.steps // 4), 5, cpu_timing=not args.no_cpu_baseline)
        torch.cuda.empty_cache()
        result["agentkv_select"] = bench_select(20, 3)
        torch.cuda.empty_cache()
        result["akv"] = bench_akv(max(20, args.steps // 4), 5, cpu_timing=not args.no_cpu_baseline)
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sc, args.cpu_budget)
        if not args.only_decode:
            result["cpu_baseline"]["oracle_full_tiny_fork"] = oracle_full_timing(
                W.tiny_fork(), "every branch of the tiny fp32 fork workload")
    if ceilings and "prefill" in result:
        r = result["prefill"]["roofline"]
        r["frac_of_measured_mfma_ceiling"] = r["achieved"] / ceilings["mfma_bf16"]["TFLOPs"]
    if ceilings and "akv" in result:
        c = result["akv"]["compaction"]
        c["frac_of_measured_copy_ceiling"] = c["GBps"] / ceilings["copy_1GiB"]["GBps_read_plus_write"]
    print(json.dumps(result))


def prefill_cpu_baseline(pi, host, budget_s):
    """fp64 oracle on the packed DAG prefill: query rows drawn uniformly at random
    (seeded) until budget_s of oracle work is spent; the full run's time is estimated as
    the mean time per row x T (an unbiased estimate under uniform sampling)."""
    import numpy as np
    import workloads as W
    from oracle import prefill as pf
    q_bits, k_bits, v_bits = host
    k64, v64 = W.bf16_bits_to_f64(k_bits), W.bf16_bits_to_f64(v_bits)

    class Rows:  # q rows converted to fp64 on access
        shape = q_bits.shape

        def __getitem__(self, i):
            return W.bf16_bits_to_f64(q_bits[i])

    order = np.random.default_rng(11).permutation(pi.T)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s and done < pi.T:
        pf.attend_rows(Rows(), k64, v64, pi.segments, pi.edges, [int(order[done])], pi.sm_scale)
        done += 1
    t = time.perf_counter() - t0
    t_full = t / done * pi.T
    return {"value": PREFILL_FLOPS / t_full / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "extrapolated": True, "oracle_full_run_s_estimate": t_full,
            "sample": f"{done} query rows (all {pi.n_q_heads} heads) drawn uniformly at random from the {pi.T:,} by the fp64 "
                      f"dense-masked oracle in {t:.1f} s; full run estimated as mean time per row x T"}


def cpu_baseline(sc, budget_s):
    """Time the fp64 oracle on a bounded sample of the same workload: branches are decoded
    one at a time (cycling over the workload's branches) until `budget_s` of oracle work
    has been spent."""
    import workloads as W
    from oracle import attention as att, pagetable as pt
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    log("cpu baseline: oracle replay")
    table, _ = pt.replay(sc, with_data=True, to_f64=lambda a: W.storage_to_f64(a, sc.dtype))
    q = W.storage_to_f64(sc.q, sc.dtype)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        i = done % len(sc.queries)
        att.decode(table, [sc.queries[i]], q[i:i + 1], sc.sm_scale)
        done += 1
    t = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": done / t, "unit": "branch-tokens/s", "cores": blas_threads or cores, "kind": "oracle",
            "host_cores_visible": cores,
            "sample": f"{done} branch decodes (cycling over the {len(sc.queries)} branches of the same "
                      f"workload) by the fp64 materialising oracle in {t:.1f} s; pool replay excluded"}


if __name__ == "__main__":
    main()
