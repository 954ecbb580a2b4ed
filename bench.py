"""Benchmark: paged MLA decode on one MI355X.

Headline workload (default): long-context decode, batch 16, q_len 1, 16 heads, 65,536 cached
tokens per sequence in 64-token pages of 576 bf16 (512 latent + 64 rope), random page table,
N(0,1) values, scale 1/sqrt(192), bf16 out.

A step is one mla_decode call (split-decode kernel + merge kernel) over inputs already resident
in HBM.  Prints one JSON line:
  value        = algorithmic bytes per call / wall time per call (GB/s, whole job)
  roofline     = the split-decode kernel alone: algorithmic bytes / its mean duration (HIP events
                 on the launch stream) against 8 TB/s, beside a read-only probe that streams the
                 same number of bytes into LDS with the decode's own non-temporal loads
                 (mla_stream_probe) on the same box
  timing_us    = per-call event percentiles, the cache-flushed per-call time, the device-scheduled
                 entry point (mla_decode_devplan) on the same inputs
  configs      = every workload (tiny, paged, two_token, long, ragged) with bf16 and with FP8 cache
                 rows: call and kernel time, flushed call time, GB/s and fraction of 8 TB/s, the
                 kernel's TFLOP/s and fraction of the 2.5 PFLOP/s bf16 matrix peak (the other bound
                 at 128 rows), and the counters' HBM bytes where they were taken
  compute      = the call's matrix work as TFLOP/s, and for the long workload the pages' H20 figure
                 at that shape (context only)
  cpu_baseline = the fp64 oracle on a bounded sample of the headline workload, on this host's
                 cores (context only)

Inputs: lengths and page tables follow the recipe (inputs.config_layout, the seeded numpy draws);
the cache and query values are N(0,1) drawn on the GPU with torch's generator seeded with the
workload's seed and rounded to bf16 (FP8 rows: E4M3 codes of x / 2^e per 128-column group, as in
the recipe).  Same shapes, lengths, page tables and value distribution as the recipe, drawn in
seconds instead of minutes; the parity tests use the recipe's own numpy values.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config long] [--kv bf16|fp8]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
HEADLINE_METRIC = "µs/call and achieved HBM GB/s (% of peak), MLA decode bs=16 H=16 ctx=64K"

WORKLOAD_TEXT = {
    "tiny": "MLA decode: batch 1, q_len 1, 16 heads, one contiguous 1024-token page, fp32 out",
    "paged": "paged MLA decode: batch 16, q_len 1, 16 heads, 4096 tokens each, page 64, bf16 out",
    "two_token": "paged MLA decode: batch 32, q_len 2 (no mask), 16 heads, 16384 tokens each, page 64, bf16 out",
    "long": "long-context paged MLA decode: batch 16, q_len 1, 16 heads, 65536 tokens each, page 64, bf16 out",
    "ragged": "ragged paged MLA decode: batch 64, q_len 1, 128 heads, lengths U[1024, 65536], page 64, bf16 out",
}
KERNEL_NAME = {16: "split_decode_kernel", 32: "split32_decode_kernel", 64: "wide_decode_kernel",
               128: "wide_decode_kernel"}
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak of MI355X (the second bound at 128 rows)
FLUSH_BYTES = 512 << 20          # read between calls: more than the 256 MB last-level cache


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


def flops(prob) -> float:
    """Matrix work of a call: 2 flops per multiply-add, 576 for S^T and 512 for O^T per cached
    token and query row."""
    return float(np.sum(prob.cache_seqlens)) * prob.q_len * prob.num_heads * 2 * (576 + 512)


def device_problem(name: str, kv: str, seed=None, device="cuda"):
    """The named workload with its recipe's lengths and page table and N(0,1) values drawn on the
    GPU (see the module docstring).  Returns (problem description, device tensors)."""
    import torch
    from mla_decode_attention_paged_amd import inputs as gen
    lengths, block_table, num_pages, cfg, seed = gen.config_layout(name, seed)
    B, S, H, P = cfg["batch"], cfg["q_len"], cfg["num_heads"], cfg["page_size"]
    g = torch.Generator(device=device)
    g.manual_seed(1000003 * seed + (1 if kv == "fp8" else 0))
    rows = num_pages * P
    chunk = 1 << 20
    if kv == "bf16":
        kvt = torch.empty((rows, 576), dtype=torch.bfloat16, device=device)
        for s0 in range(0, rows, chunk):
            e0 = min(rows, s0 + chunk)
            kvt[s0:e0] = torch.randn((e0 - s0, 576), generator=g, device=device).to(torch.bfloat16)
        kvt = kvt.view(num_pages, P, 576)
    else:
        kvt = torch.empty((rows, 656), dtype=torch.uint8, device=device)
        for s0 in range(0, rows, chunk):
            e0 = min(rows, s0 + chunk)
            n = e0 - s0
            x = torch.randn((n, 4, 128), generator=g, device=device)
            amax = x.abs().amax(dim=2).clamp_min(2.0 ** -100)
            scale = torch.exp2(torch.ceil(torch.log2(amax.double() / 448.0))).float()
            kvt[s0:e0, :512] = (x / scale[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, 512)
            kvt[s0:e0, 640:656] = scale.contiguous().view(torch.uint8).reshape(n, 16)
            rope = torch.randn((n, 64), generator=g, device=device).to(torch.bfloat16)
            kvt[s0:e0, 512:640] = rope.view(torch.uint8).reshape(n, 128)
        kvt = kvt.view(num_pages, P, 656)
    q = torch.randn((B, S, H, 576), generator=g, device=device).to(torch.bfloat16)
    dev = {"q": q, "kv_cache": kvt, "block_table": torch.from_numpy(block_table).to(device),
           "cache_seqlens": torch.from_numpy(lengths).to(device)}
    prob = SimpleNamespace(name=name, batch=B, q_len=S, num_heads=H, page_size=P, num_pages=num_pages,
                           max_pages_per_seq=int(block_table.shape[1]), out_fp32=bool(cfg.get("out_fp32", False)),
                           kv_format=kv, cache_seqlens=lengths, block_table=block_table,
                           softmax_scale=gen.SOFTMAX_SCALE, seed=seed)
    return prob, dev


def measured_traffic(key: str):
    """HBM bytes per split-decode launch from the committed counter summary, or None when the
    summary is missing, for another workload, or older than the kernel sources."""
    try:
        with open(PROFILE_COUNTERS) as fh:
            c = json.load(fh)
    except (OSError, ValueError):
        return None
    from mla_decode_attention_paged_amd.profiling import kernel_source_hash
    entry = c.get(key)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_runner(r, stream, steps: int, flush=None, flushed_calls: int = 10):
    """(mean us per call back-to-back, mean us of the split kernel alone, p50 us per call after
    reading `flush` between calls)."""
    import torch
    from mla_decode_attention_paged_amd import binding as B
    e0, e1 = _events()
    e0.record(stream)
    for _ in range(steps):
        r()
    e1.record(stream)
    torch.cuda.synchronize()
    call = e0.elapsed_time(e1) * 1e3 / steps
    e0, e1 = _events()
    e0.record(stream)
    for _ in range(steps):
        r(stages=B.MLA_STAGE_SPLIT)
    e1.record(stream)
    torch.cuda.synchronize()
    kern = e0.elapsed_time(e1) * 1e3 / steps
    fl = []
    if flush is not None:
        for _ in range(flushed_calls):
            flush.sum()
            a, b = _events()
            a.record(stream)
            r()
            b.record(stream)
            torch.cuda.synchronize()
            fl.append(a.elapsed_time(b) * 1e3)
    return call, kern, (float(np.median(fl)) if fl else None)


def config_table(stream, flush, steps: int = 20, warm_ms: float = 100.0, rep_ms: float = 20.0, reps: int = 3):
    """Every workload with bf16 and FP8 cache rows.  Each is warmed up for about `warm_ms` of
    back-to-back calls (the first tens of calls after a switch of workload run slower while the
    clocks settle), then timed `reps` times over at least `steps` calls and `rep_ms`; the
    medians of the reps are reported."""
    import torch
    from mla_decode_attention_paged_amd.device import Runner
    from mla_decode_attention_paged_amd import inputs as gen
    table = {}
    for name in gen.CONFIG_ORDER:
        for kv in ("bf16", "fp8"):
            print(f"[bench] config {name} {kv}", file=sys.stderr, flush=True)
            prob, dev = device_problem(name, kv)
            r = Runner(prob, dev=dev)
            info = r.plan.info()
            for _ in range(10):
                r()
            e0, e1 = _events()
            e0.record(stream)
            for _ in range(10):
                r()
            e1.record(stream)
            torch.cuda.synchronize()
            per_call_ms = max(e0.elapsed_time(e1) / 10, 1e-3)
            for _ in range(max(30, int(warm_ms / per_call_ms))):
                r()
            n = max(steps, int(rep_ms / per_call_ms))
            runs = [time_runner(r, stream, n) for _ in range(reps)]
            call = float(np.median([x[0] for x in runs]))
            kern = float(np.median([x[1] for x in runs]))
            flushed = time_runner(r, stream, 1, flush)[2]
            algo = algorithmic_bytes(prob)
            entry = {
                "us_per_call": round(call, 2), "kernel_us": round(kern, 2), "call_flushed_us": round(flushed, 2),
                "algorithmic_bytes": algo,
                "GBps_kernel": round(algo / (kern * 1e-6) / 1e9, 1),
                "GBps_call_flushed": round(algo / (flushed * 1e-6) / 1e9, 1),
                "frac_kernel": round(algo / (kern * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "frac_call_flushed": round(algo / (flushed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "kernel_tflops": round(flops(prob) / (kern * 1e-6) / 1e12, 1),
                "frac_mfma_kernel": round(flops(prob) / (kern * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                "kernel": KERNEL_NAME[info["rows_per_group"]], "rows_per_group": info["rows_per_group"],
                "row_groups": info["row_groups"], "pieces": info["num_segments"], "partials": info["num_partials"],
            }
            traffic = measured_traffic(name if kv == "bf16" else f"{name}_fp8")
            entry["traffic"] = traffic
            table[f"{name}_{kv}"] = entry
            del r, dev
            torch.cuda.empty_cache()
    return table


def read_probe(stream, nbytes: int, grid: int, reps: int = 10):
    """Best-of-reps GB/s of mla_stream_probe over a buffer of nbytes on `grid` work-groups."""
    import torch
    from mla_decode_attention_paged_amd import binding as B
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    B.mla_stream_probe(buf, grid)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        a, b = _events()
        a.record(stream)
        B.mla_stream_probe(buf, grid)
        b.record(stream)
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3
        best = t if best is None else min(best, t)
    unit = 73728 * grid
    moved = nbytes // unit * unit
    del buf
    return moved / best / 1e9


def cpu_baseline(prob, dev, budget_s: float = 15.0):
    """Time the oracle on whole sequences of the workload (copied to the host) until about
    budget_s seconds."""
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    q = dev["q"].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    kv = dev["kv_cache"]
    kv_host = (kv.cpu().numpy() if prob.kv_format == "fp8"
               else kv.view(__import__("torch").int16).cpu().numpy().view(np.uint16))
    done, t_total, tokens = [], 0.0, 0
    for b in range(prob.batch):
        t0 = time.perf_counter()
        orc.decode_sequence(q[b], kv_host, prob.block_table[b], int(prob.cache_seqlens[b]), prob.softmax_scale,
                            prob.page_size)
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
            a, b = _events()
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / reps)
        res[name] = float(np.median(times))
        del g
    nb = layer_bytes(prob)
    return {"us": {k: round(v, 2) for k, v in res.items()},
            "algorithmic_bytes": nb,
            "GBps": {k: round(nb[k] / (res[k] * 1e-6) / 1e9, 1) for k in nb},
            "note": "graph-replayed means over back-to-back launches; the layer step is append + query "
                    "preparation + decode + output projection"}


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
    ap.add_argument("--no-configs", action="store_true", help="skip the table of every workload")
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
    from mla_decode_attention_paged_amd.device import DevplanRunner, Runner, problem_struct
    from mla_decode_attention_paged_amd.profiling import kernel_source_hash

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()  # fail loudly if the HIP library is missing
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"[bench] generating {args.config} inputs ({args.kv} cache) on the GPU", file=sys.stderr, flush=True)
    prob, dev = device_problem(args.config, args.kv, args.seed)
    algo = algorithmic_bytes(prob)
    counters_key = args.config if args.kv == "bf16" else f"{args.config}_{args.kv}"

    t0 = time.perf_counter()
    plan_probe = B.Plan(problem_struct(prob), prob.cache_seqlens)
    plan_us = (time.perf_counter() - t0) * 1e6
    del plan_probe
    r = Runner(prob, dev=dev)
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

    # per-call event timing (same stream), the split-decode kernel alone, and flushed calls
    ev = [_events() for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        r()
        b.record(stream)
    torch.cuda.synchronize()
    call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    _, split_us, flushed_us = time_runner(r, stream, args.steps, flush, min(args.steps, 20))
    status = B.mla_read_status(r.ws)

    # the same workload through the device-scheduled entry point (no host plan)
    dr = DevplanRunner(prob, dev=r.dev)
    for _ in range(10):
        dr()
    torch.cuda.synchronize()
    d0, d1 = _events()
    d0.record(stream)
    for _ in range(args.steps):
        dr()
    d1.record(stream)
    torch.cuda.synchronize()
    devplan_us = d0.elapsed_time(d1) * 1e3 / args.steps
    del dr

    # read ceiling: the decode's KV bytes streamed into LDS by the same loads, same grid size
    print("[bench] read probe", file=sys.stderr, flush=True)
    kv_bytes = int(np.sum(prob.cache_seqlens)) * (656 if args.kv == "fp8" else 1152)
    probe_gbs = read_probe(stream, max(kv_bytes, 73728 * cus), cus)

    layer = None
    if not args.no_layer:
        print("[bench] timing the steps around the decode", file=sys.stderr, flush=True)
        layer = layer_leg(prob, r)

    table = None
    if not args.no_configs:
        table = config_table(stream, flush)
    del flush

    value = algo / wall / 1e9
    achieved = algo / (split_us * 1e-6) / 1e9
    traffic = measured_traffic(counters_key)
    fl = flops(prob)
    compute = {"flops_per_call": fl, "kernel_tflops": round(fl / (split_us * 1e-6) / 1e12, 1),
               "call_tflops": round(fl / wall / 1e12, 1)}
    if args.config == "long":
        compute["pages_figure"] = ("FlashMLA-ETAP 89 TFLOP/s against FlashMLA 32 TFLOP/s (2.78x) at 64K tokens, "
                                   "batch 16, on an NVIDIA H20 ([ETAP] 'Experimental results'); not comparable")
    metric = HEADLINE_METRIC if args.config == "long" else \
        f"µs/call and achieved HBM GB/s (% of peak), {WORKLOAD_TEXT[args.config]}"
    result = {
        "metric": metric,
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
                   "parallelism": f"single GPU, split-KV over {cus} CUs",
                   "arithmetic": "bf16 matrix products with fp32 accumulation (FP8 rows widened to bf16 exactly)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": KERNEL_NAME[info["rows_per_group"]],
                     "kernel_us": round(split_us, 2),
                     "algorithmic_bytes_per_launch": algo,
                     "read_probe_GBps": round(probe_gbs, 1),
                     "frac_of_read_probe": round(achieved / probe_gbs, 4)},
        "timing_us": {"call_event_p10": round(float(np.percentile(call_us, 10)), 2),
                      "call_event_p50": round(float(np.percentile(call_us, 50)), 2),
                      "call_event_p90": round(float(np.percentile(call_us, 90)), 2),
                      "call_flushed_p50": round(flushed_us, 2),
                      "split_kernel_mean": round(split_us, 2),
                      "merge_and_gap_p50": round(float(np.percentile(call_us, 50)) - split_us, 2),
                      "plan_host_us": round(plan_us, 1),
                      "devplan_call_mean": round(devplan_us, 2)},
        "plan": {k: info[k] for k in ("num_workers", "grid_size", "num_segments", "num_partials", "num_combine",
                                      "rows_per_group", "row_groups")},
        "status_word": status,
        "kernel_source_hash": kernel_source_hash(),
        "compute": compute,
        "configs": table,
        "layer_steps": layer,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(prob, r.dev, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
