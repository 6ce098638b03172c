"""Benchmark: one step = one fork_attn_decode over every branch of the shared-prefix fork
workload (16 branches x 32 query heads, 8 KV heads, d=128, bf16, 32,768-token shared
prefix + 2,048 private tokens per branch, page 16), inputs resident in HBM.

Prints ONE JSON line.  `value` = branch-tokens/s (branches decoded per second, wall clock
over the timed steps); the roofline object prices the dominant kernel (decode_kernel)
against MI355X's 8 TB/s HBM with its algorithmic bytes (unique KV + Q), timed with HIP
events on the launch stream; `step` reports the whole step (decode + merge) the same way.  Steps rotate over
several identical pool copies so that no step finds its KV in the 256 MB last-level
cache left behind by the previous one.  The cpu_baseline leg times the fp64 oracle on a
bounded sample of the same workload on the host cores.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_traffic.json")


def measured_traffic():
    """HBM bytes per decode_kernel launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs, or None once the kernel sources differ from the profiled ones."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        h = hashlib.sha256()
        for f in rec["source_files"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["source_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4, help="pool copies rotated between steps")
    ap.add_argument("--workload", default="shared_prefix_fork_decode",
                    choices=["shared_prefix_fork_decode", "octopus_dag_decode", "tiny_fork_decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work to sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, copy 256 MiB device to device once (a kernel of known "
                         "traffic to scale hardware byte counters against)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this build runs on "
              f"a single MI355X; decode shards by KV head with no exchange across GPUs).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    import fork_attention_decode_amd as fa
    from tests.harness import build_device_pool, to_torch

    torch.cuda.set_device(0)
    sc = W.WORKLOADS[args.workload]()
    print(f"[bench] workload {args.workload}: building {args.copies} pool copies", file=sys.stderr, flush=True)
    pools = [build_device_pool(sc)[0] for _ in range(args.copies)]
    q = to_torch(sc.q, sc.dtype)
    n_br, hq, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((n_br, hq), dtype=torch.float32, device=q.device)
    wss = []
    for p in pools:
        need = fa.fork_attn_workspace_size(p.handle, sc.queries, hq)
        wss.append(torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device))
    stats = pools[0].plan_stats()
    es = 2 if sc.dtype == "bf16" else 4
    kernel_bytes = stats["unique_kv_bytes"] + q.numel() * es   # decode kernel: unique KV + Q read
    step_bytes = kernel_bytes + q.numel() * es                 # whole step: + O written by the merge
    stream = torch.cuda.current_stream().cuda_stream

    def step(i, ev=None):
        # one step = the decode kernel (partials) + the merge kernel; events on the
        # launch stream bracket the decode kernel alone and the whole step
        p = pools[i % len(pools)]
        ws = wss[i % len(pools)]
        if ev:
            ev[0].record()
        fa.fork_attn_partials(p.handle, sc.queries, hq, q.data_ptr(), sc.sm_scale, ws.data_ptr(), ws.numel(), stream)
        if ev:
            ev[1].record()
        fa.fork_attn_merge(p.handle, sc.queries, hq, out.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        if ev:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=q.device)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    k_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])      # decode kernel
    s_ms = np.array([a.elapsed_time(c) for a, _, c in ev])      # whole step (decode + merge)
    ms_step = wall * 1e3 / args.steps
    t_kernel = float(np.mean(k_ms)) * 1e-3
    achieved = kernel_bytes / t_kernel / 1e9

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
                   "head_dim": d, "page_size": sc.page_size, "pool_copies_rotated": args.copies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic() if args.workload == "shared_prefix_fork_decode" else None,
                     "kernel": "decode_kernel (fork_attn_partials)",
                     "algorithmic_bytes_per_launch": kernel_bytes,
                     "kernel_us_mean": float(np.mean(k_ms)) * 1e3,
                     "kernel_us_p10": float(np.percentile(k_ms, 10)) * 1e3,
                     "kernel_us_p90": float(np.percentile(k_ms, 90)) * 1e3},
        "step": {"us_mean_events": float(np.mean(s_ms)) * 1e3, "algorithmic_bytes": step_bytes,
                 "achieved_GBps": step_bytes / (float(np.mean(s_ms)) * 1e-3) / 1e9,
                 "frac_of_peak": step_bytes / (float(np.mean(s_ms)) * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                 "merge_us_mean": float(np.mean(s_ms - k_ms)) * 1e3},
        "plan": stats,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sc, args.cpu_budget)
    print(json.dumps(result))


def cpu_baseline(sc, budget_s):
    """Time the fp64 oracle on a bounded sample of the same workload: branches are decoded
    one at a time (cycling over the workload's branches) until `budget_s` of oracle work
    has been spent."""
    import numpy as np
    import workloads as W
    from oracle import attention as att, pagetable as pt
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    print("[bench] cpu baseline: oracle replay", file=sys.stderr, flush=True)
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
