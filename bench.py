"""Benchmark: paged MLA decode on one MI355X.

Workload (default): long-context decode, batch 16, q_len 1, 16 heads, 65,536
cached tokens per sequence in 64-token pages of 576 bf16 (512 latent + 64
rope), random page table, N(0,1) values, scale 1/sqrt(192), bf16 out.

A step is one mla_decode call (split-decode kernel + merge kernel) over inputs
already resident in HBM.  Prints one JSON line:
  value      = algorithmic bytes per call / wall time per call  (GB/s, whole job)
  roofline   = the split-decode kernel alone: algorithmic bytes / its mean
               duration (HIP events on the launch stream) vs 8 TB/s HBM, and vs
               a 1 GiB device-to-device copy timed on the same box
  timing_us  = per-call event percentiles, the cache-flushed per-call time, the
               device-scheduled entry point (mla_decode_devplan) on the same inputs
  compute    = the call's matrix work as TFLOP/s (kernel and whole call), and for
               the long workload the pages' H20 figure at that shape (context only)
  cpu_baseline = the fp64 oracle on a bounded sample of the same workload, on
               this host's cores (context only)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config long]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "counters.json")

WORKLOAD_TEXT = {
    "tiny": "MLA decode: batch 1, q_len 1, 16 heads, one contiguous 1024-token page, fp32 out",
    "paged": "paged MLA decode: batch 16, q_len 1, 16 heads, 4096 tokens each, page 64, bf16 out",
    "two_token": "paged MLA decode: batch 32, q_len 2 (no mask), 16 heads, 16384 tokens each, page 64, bf16 out",
    "long": "long-context paged MLA decode: batch 16, q_len 1, 16 heads, 65536 tokens each, page 64, bf16 out",
    "ragged": "ragged paged MLA decode: batch 64, q_len 1, 128 heads, lengths U[1024, 65536], page 64, bf16 out",
}


def algorithmic_bytes(prob) -> int:
    """Bytes the decode must move at least once: every cached row once (K and V share it),
    the query, the output, the lse, and the used block-table entries."""
    L = prob.cache_seqlens.astype(np.int64)
    R = prob.q_len * prob.num_heads
    out_elem = 4 if prob.out_fp32 else 2
    row_bytes = 656 if prob.kv_format == "fp8" else 576 * 2
    pages = ((L + prob.page_size - 1) // prob.page_size).sum()
    return int(L.sum() * row_bytes + prob.batch * R * 576 * 2 + prob.batch * R * 512 * out_elem
               + prob.batch * R * 4 + pages * 4)


def measured_traffic(config: str):
    """HBM bytes per split-decode launch from the committed counter summary, or None when
    the summary is missing, for another workload, or older than the kernel sources."""
    try:
        with open(PROFILE_COUNTERS) as fh:
            c = json.load(fh)
    except (OSError, ValueError):
        return None
    from mla_decode_attention_paged_amd.profiling import kernel_source_hash
    entry = c.get(config)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def compute_context(prob, kernel_us: float, call_s: float, config: str):
    """Matrix work of the call (2 flops per multiply-add: 576 for S^T and 512 for O^T per
    cached token and query row) as a rate, and, for the long workload, the pages' figure at
    the same shape on other hardware (context only: another GPU, another flop count may be
    meant)."""
    R = prob.q_len * prob.num_heads
    flops = float(np.sum(prob.cache_seqlens)) * R * 2 * (576 + 512)
    out = {"flops_per_call": flops,
           "kernel_tflops": round(flops / (kernel_us * 1e-6) / 1e12, 1),
           "call_tflops": round(flops / call_s / 1e12, 1)}
    if config == "long":
        out["pages_figure"] = ("FlashMLA-ETAP 89 TFLOP/s against FlashMLA 32 TFLOP/s (2.78x) at 64K tokens, "
                               "batch 16, on an NVIDIA H20 ([ETAP] 'Experimental results'); not comparable")
    return out


def cpu_baseline(prob, budget_s: float = 15.0):
    """Time the oracle on whole sequences of the workload until about budget_s seconds."""
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    order = list(range(prob.batch))
    done, t_total, tokens, rows_bytes = [], 0.0, 0, 0
    for b in order:
        t0 = time.perf_counter()
        orc.decode_sequence(prob.q[b], prob.kv_cache, prob.block_table[b], int(prob.cache_seqlens[b]),
                            prob.softmax_scale, prob.page_size)
        t_total += time.perf_counter() - t0
        done.append(b)
        tokens += int(prob.cache_seqlens[b])
        if t_total >= budget_s:
            break
    frac = tokens / max(1, int(prob.cache_seqlens.sum()))
    sample_bytes = algorithmic_bytes(prob) * frac
    return {
        "value": round(sample_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(done)} of {prob.batch} sequences ({tokens} tokens, {100 * frac:.1f}% of the call), "
                  f"fp64 NumPy, {t_total:.2f} s; extrapolated {t_total / frac * 1e6:.0f} us/call",
        "us_per_call_extrapolated": round(t_total / frac * 1e6, 1),
    }


ROPE_BASE = 10000.0


def layer_bytes(prob) -> dict:
    """Algorithmic bytes of the steps around the decode (each input and output once)."""
    n, H = prob.batch * prob.q_len, prob.num_heads
    out_elem = 4 if prob.out_fp32 else 2
    row_bytes = 656 if prob.kv_format == "fp8" else 576 * 2
    return {
        "q_absorb": H * 512 * 128 * 2 + n * H * (128 + 64) * 2 + n * 4 + n * H * 576 * 2,
        "kv_append": n * (512 + 64) * 2 + n * 8 + n * row_bytes,
        "out_absorb": H * 128 * 512 * 2 + n * H * 512 * out_elem + n * H * 128 * out_elem,
    }


def layer_leg(prob, r, reps: int = 20):
    """Mean device time of each step around the decode, and of one whole layer step
    (append, query preparation, decode, output projection), from HIP graphs of `reps`
    back-to-back launches replayed on the current stream (no host time in the figures).
    Runs after the decode timing: the append rewrites each sequence's last row."""
    import torch
    from mla_decode_attention_paged_amd import binding as B
    from mla_decode_attention_paged_amd import inputs as gen
    from mla_decode_attention_paged_amd.device import layer_to_device, problem_struct
    li = gen.make_layer_inputs(prob.batch, prob.q_len, prob.num_heads, seed=prob.seed + 1000)
    d = layer_to_device(li)
    p = problem_struct(prob)
    pos = torch.from_numpy((prob.cache_seqlens[:, None] - prob.q_len
                            + np.arange(prob.q_len)[None, :]).astype(np.int32)).cuda()
    odt = torch.float32 if prob.out_fp32 else torch.bfloat16
    o = torch.empty((prob.batch, prob.q_len, prob.num_heads, 128), dtype=odt, device="cuda")
    dev = r.dev
    steps = {
        "q_absorb": lambda: B.mla_q_absorb(p, d["q_nope"], d["q_pe"], d["w_uk"], pos, ROPE_BASE, dev["q"]),
        "kv_append": lambda: B.mla_kv_append(p, d["c_kv"], d["k_pe"], pos, dev["block_table"], ROPE_BASE,
                                             dev["kv_cache"]),
        "out_absorb": lambda: B.mla_out_absorb(p, r.out, d["w_uv"], o),
    }

    def whole():
        steps["kv_append"]()
        steps["q_absorb"]()
        r()
        steps["out_absorb"]()
    steps["layer_step"] = whole
    res = {}
    stream = torch.cuda.current_stream()
    for name, fn in steps.items():
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / reps)
        res[name] = float(np.median(times))
        del g
    nb = layer_bytes(prob)
    out = {"us": {k: round(v, 2) for k, v in res.items()},
           "algorithmic_bytes": nb,
           "GBps": {k: round(nb[k] / (res[k] * 1e-6) / 1e9, 1) for k in nb},
           "note": "graph-replayed means over back-to-back launches; the layer step is append + query "
                   "preparation + decode + output projection"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", default="long", choices=list(WORKLOAD_TEXT))
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-layer", action="store_true", help="skip timing the steps around the decode")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="cache row storage: bf16 (1,152 B per token) or fp8 E4M3 rows (656 B per token)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the library runs the decode "
              "on a single MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_decode_attention_paged_amd import binding as B
    from mla_decode_attention_paged_amd import inputs as gen
    from mla_decode_attention_paged_amd.device import Runner

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()  # fail loudly if the HIP library is missing
    print(f"[bench] generating {args.config} inputs", file=sys.stderr, flush=True)
    prob = gen.make_config(args.config, seed=args.seed, kv_format=args.kv)
    algo = algorithmic_bytes(prob)
    counters_key = args.config if args.kv == "bf16" else f"{args.config}_{args.kv}"

    t0 = time.perf_counter()
    plan_probe = B.Plan(__import__("mla_decode_attention_paged_amd.device", fromlist=["x"]).problem_struct(prob),
                        prob.cache_seqlens)
    plan_us = (time.perf_counter() - t0) * 1e6
    del plan_probe
    r = Runner(prob)
    stream = torch.cuda.current_stream()
    info = r.plan.info()

    for _ in range(args.warmup):
        r()
    torch.cuda.synchronize()

    # whole-call throughput: K back-to-back calls
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        r()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps

    # per-call event timing (same stream), and the split-decode kernel alone
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        r()
        b.record(stream)
    torch.cuda.synchronize()
    call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        r(stages=B.MLA_STAGE_SPLIT)
    e1.record(stream)
    torch.cuda.synchronize()
    split_us = e0.elapsed_time(e1) * 1e3 / args.steps

    # flushed per-call time: reading 512 MB between calls evicts the 256 MB last-level cache
    # (a read, so no dirty lines are left to be written back during the timed call)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    fl = []
    for _ in range(min(args.steps, 20)):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        r()
        b.record(stream)
        torch.cuda.synchronize()
        fl.append(a.elapsed_time(b) * 1e3)
    del flush

    status = B.mla_read_status(r.ws)

    # the same workload through the device-scheduled entry point (no host plan); FP8 and
    # every R run there on the 16-row kernel
    from mla_decode_attention_paged_amd.device import DevplanRunner
    dr = DevplanRunner(prob, dev=r.dev)
    for _ in range(10):
        dr()
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(args.steps):
        dr()
    d1.record(stream)
    torch.cuda.synchronize()
    devplan_us = d0.elapsed_time(d1) * 1e3 / args.steps
    del dr

    # read-bandwidth reference on this machine: a 1 GiB device-to-device copy (reads 1 GiB,
    # writes 1 GiB), best of 10
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    cps = []
    for _ in range(10):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        cps.append(c0.elapsed_time(c1) * 1e-3)
    copy_gbs = 2 * src.numel() * 4 / min(cps) / 1e9
    del src, dst

    layer = None
    if not args.no_layer:
        print("[bench] timing the steps around the decode", file=sys.stderr, flush=True)
        layer = layer_leg(prob, r)
    value = algo / wall / 1e9
    achieved = algo / (split_us * 1e-6) / 1e9
    traffic = measured_traffic(counters_key)
    result = {
        "metric": "µs/call and achieved HBM GB/s (% of peak), MLA decode bs=16 H=16 ctx=64K",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 5),
        "us_per_call": round(wall * 1e6, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config] + ("" if args.kv == "bf16" else
                                                             ", FP8 E4M3 cache rows (656 B per token)"),
                   "name": args.config, "kv": args.kv, "batch": prob.batch,
                   "q_len": prob.q_len, "heads": prob.num_heads, "page_size": prob.page_size,
                   "ctx_tokens_total": int(prob.cache_seqlens.sum()), "seed": prob.seed,
                   "parallelism": "single GPU, split-KV over 256 CUs"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "split_decode_kernel" if info["rows_per_group"] == 16 else "group_decode_kernel",
                     "kernel_us": round(split_us, 2),
                     "algorithmic_bytes_per_launch": algo,
                     "copy_probe_GBps": round(copy_gbs, 1),
                     "frac_of_copy_probe": round(achieved / copy_gbs, 4)},
        "timing_us": {"call_event_p10": round(float(np.percentile(call_us, 10)), 2),
                      "call_event_p50": round(float(np.percentile(call_us, 50)), 2),
                      "call_event_p90": round(float(np.percentile(call_us, 90)), 2),
                      "call_flushed_p50": round(float(np.median(fl)), 2),
                      "split_kernel_mean": round(split_us, 2),
                      "merge_and_gap_p50": round(float(np.percentile(call_us, 50)) - split_us, 2),
                      "plan_host_us": round(plan_us, 1),
                      "devplan_call_mean": round(devplan_us, 2)},
        "plan": {k: info[k] for k in ("num_workers", "grid_size", "num_segments", "num_partials", "num_combine")},
        "status_word": status,
        "compute": compute_context(prob, split_us, wall, args.config),
        "layer_steps": layer,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(prob, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
