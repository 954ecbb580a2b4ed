"""rocprofv3 helpers: a copy kernel of known size (counter calibration) and summaries.

rocprofv3 writes one SQLite database (<pid>_results.db) per profiled process; the
summaries below read its `top_kernels` and `counters_collection` views.

  python -m mla_decode_attention_paged_amd.profiling calib
      device-to-device copy of 1 GiB, 5 times (run it under `rocprofv3 --pmc ...`)
  python -m mla_decode_attention_paged_amd.profiling stats DIR OUT.md "COMMAND"
      summarise a `rocprofv3 --kernel-trace --stats` output directory
  python -m mla_decode_attention_paged_amd.profiling counters CONFIG KERNEL FETCH_DIR WRITE_DIR \
         CALIB_FETCH_DIR CALIB_WRITE_DIR OUT.md "COMMANDS"
      HBM bytes per launch of KERNEL from FETCH_SIZE / WRITE_SIZE passes, each scaled by
      what the same counter reads for the 1 GiB copy; updates profiles/counters.json
  python -m mla_decode_attention_paged_amd.profiling sq KERNEL BLOCKS OUT.md "COMMANDS" DIR [DIR ...]
      mean SQ counters per dispatch of KERNEL over `rocprofv3 --pmc SQ_...` passes
"""
from __future__ import annotations

import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CALIB_BYTES = 1 << 30
KERNEL_SOURCES = [os.path.join(HERE, "csrc", f) for f in ("mla_kernels.hip", "mla_internal.h", "plan.cpp",
                                                          "mla_api.cpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def calib(reps: int = 5):
    import torch
    n = CALIB_BYTES // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {CALIB_BYTES} bytes x {reps}", flush=True)


def _dbs(d):
    files = sorted(glob.glob(os.path.join(d, "**", "*results.db"), recursive=True))
    if not files:
        raise SystemExit(f"no rocprofv3 results.db under {d}")
    return files


def _short(name):
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")[:80]


def stats(d, out_md, command):
    """Per-kernel duration statistics from the dispatch records (kernel trace)."""
    import sqlite3
    agg = {}
    for f in _dbs(d):
        con = sqlite3.connect(f)
        for name, dur in con.execute("select name, duration from kernels"):
            agg.setdefault(name, []).append(dur / 1e3)
        con.close()
    total = sum(sum(v) for v in agg.values())
    lines = ["# rocprofv3 kernel statistics", "", f"Kernel source hash: {kernel_source_hash()}", "",
             "Command (run from /tmp with TMPDIR=/tmp):", "", "```", command,
             "```", "", "| kernel | calls | avg us | min us | max us | total us | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for name, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{_short(name)}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{sum(v):.1f} | {100 * sum(v) / total:.2f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_per_dispatch(d, counter, kernel_substr):
    import sqlite3
    vals = {}
    for f in _dbs(d):
        con = sqlite3.connect(f)
        for disp, kname, cname, value in con.execute(
                "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
            if cname != counter or kernel_substr not in kname:
                continue
            vals[(f, disp)] = vals.get((f, disp), 0.0) + float(value)
        con.close()
    return list(vals.values()), None


def counters(config, kernel, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, out_md, commands):
    f, _ = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", kernel)
    w, _ = _counter_per_dispatch(write_dir, "WRITE_SIZE", kernel)
    cf, _ = _counter_per_dispatch(cal_fetch_dir, "FETCH_SIZE", "")
    cw, _ = _counter_per_dispatch(cal_write_dir, "WRITE_SIZE", "")
    # the copy kernel: the dispatches with the largest counter values
    cf_v = max(cf) if cf else 0.0
    cw_v = max(cw) if cw else 0.0
    if not f or not w or cf_v <= 0 or cw_v <= 0:
        raise SystemExit(f"missing counters: fetch {len(f)} write {len(w)} calib {cf_v} {cw_v}")
    fetch_scale = CALIB_BYTES / (cf_v * 1024.0)
    write_scale = CALIB_BYTES / (cw_v * 1024.0)
    fetch_kib = sum(f) / len(f)
    write_kib = sum(w) / len(w)
    fetch_b = fetch_kib * 1024.0 * fetch_scale
    write_b = write_kib * 1024.0 * write_scale
    entry = {"kernel": kernel, "dispatches": [len(f), len(w)], "fetch_kib_per_dispatch": fetch_kib,
             "write_kib_per_dispatch": write_kib, "calib_fetch_kib": cf_v, "calib_write_kib": cw_v,
             "fetch_scale": fetch_scale, "write_scale": write_scale,
             "hbm_bytes_per_launch": round(fetch_b + write_b), "fetch_bytes_per_launch": round(fetch_b),
             "write_bytes_per_launch": round(write_b), "kernel_source_hash": kernel_source_hash()}
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as fh:
            allc = json.load(fh)
    except (OSError, ValueError):
        allc = {}
    allc[config] = entry
    with open(path, "w") as fh:
        json.dump(allc, fh, indent=1, sort_keys=True)
    lines = [f"# HBM traffic of `{kernel}` ({config} workload)", "", "Commands:", "", "```", commands, "```", "",
             f"- FETCH_SIZE: {fetch_kib:.0f} KiB per dispatch ({len(f)} dispatches); the 1 GiB copy reads "
             f"{cf_v:.0f} KiB, so scale x{fetch_scale:.4f} -> {fetch_b / 1e6:.2f} MB per launch",
             f"- WRITE_SIZE: {write_kib:.0f} KiB per dispatch ({len(w)} dispatches); the 1 GiB copy writes "
             f"{cw_v:.0f} KiB, so scale x{write_scale:.4f} -> {write_b / 1e6:.2f} MB per launch",
             f"- HBM traffic per launch: {(fetch_b + write_b) / 1e6:.2f} MB",
             f"- kernel source hash: {entry['kernel_source_hash']}"]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def sq(kernel, blocks, out_md, commands, *dirs):
    """Mean per dispatch of every SQ counter found in the `rocprofv3 --pmc` directories, for
    dispatches whose kernel name contains `kernel`; with `blocks` (16-token block visits per
    launch, 16 rows each) also instructions per block.  Derived: MFMA busy share of the wave
    cycles (SQ_WAVE_CYCLES counts in units of 4 cycles; one wave per SIMD)."""
    import sqlite3
    sums, disp = {}, {}
    for d in dirs:
        for f in _dbs(d):
            con = sqlite3.connect(f)
            for dsp, kname, cname, value in con.execute(
                    "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
                if kernel not in kname or not cname.startswith("SQ_"):
                    continue
                sums[cname] = sums.get(cname, 0.0) + float(value)
                disp.setdefault(cname, set()).add((f, dsp))
            con.close()
    if not sums:
        raise SystemExit(f"no SQ counters for {kernel}")
    mean = {c: sums[c] / len(disp[c]) for c in sums}
    blocks = int(blocks)
    lines = [f"# SQ counters of `{kernel}`", "", f"Kernel source hash: {kernel_source_hash()}", "",
             "Commands (run from /tmp with TMPDIR=/tmp):", "", "```", commands, "```",
             "", "| counter | mean per dispatch | per block |", "|---|---|---|"]
    for c in sorted(mean):
        per = f"{mean[c] / blocks:.1f}" if blocks > 0 else ""
        lines.append(f"| {c} | {mean[c]:.0f} | {per} |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "SQ_WAVE_CYCLES" in mean:
        lines += ["", f"- MFMA busy / wave cycles: {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * mean['SQ_WAVE_CYCLES']):.3f}"]
    if blocks > 0 and "SQ_WAVE_CYCLES" in mean:
        lines += [f"- wave cycles per block visit: {4 * mean['SQ_WAVE_CYCLES'] / blocks:.0f}"]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    cmd = sys.argv[1]
    if cmd == "calib":
        calib()
    elif cmd == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif cmd == "counters":
        counters(*sys.argv[2:10])
    elif cmd == "sq":
        sq(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
