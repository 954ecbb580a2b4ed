"""Host-side parts of bench.py (no GPU): the byte and flop counts behind `value` and `roofline`,
the counter lookup that fills `traffic`, and the one-GPU guard."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mla_decode_attention_paged_amd import inputs as gen  # noqa: E402


def workload(name, kv="bf16"):
    lengths, block_table, num_pages, cfg, seed = gen.config_layout(name)
    return SimpleNamespace(batch=cfg["batch"], q_len=cfg["q_len"], num_heads=cfg["num_heads"],
                           page_size=cfg["page_size"], out_fp32=bool(cfg.get("out_fp32", False)), kv_format=kv,
                           cache_seqlens=np.asarray(lengths, dtype=np.int32))


def test_long_workload_bytes_and_flops():
    """16 sequences of 65,536 tokens, 16 heads: 1,152 B per cached row read once, plus the query
    (16 x 16 rows x 1,152 B), the bf16 output (x 1,024 B), the lse (x 4 B) and 1,024 table
    entries per sequence; 2 x (576 + 512) flops per cached token and query row."""
    p = workload("long")
    kv = 16 * 65536 * 1152
    assert kv == 1_207_959_552
    assert bench.algorithmic_bytes(p) == kv + 256 * 1152 + 256 * 1024 + 256 * 4 + 16 * 1024 * 4 == 1_208_583_168
    assert bench.flops(p) == 16 * 65536 * 16 * 2 * 1088
    f8 = workload("long", "fp8")
    assert bench.algorithmic_bytes(f8) == 16 * 65536 * 656 + 256 * 1152 + 256 * 1024 + 256 * 4 + 16 * 1024 * 4


def test_tiny_and_ragged_bytes():
    """The tiny workload writes fp32 (2,048 B per row) from one 1,024-token page; the ragged one
    counts each sequence's own length and pages of 64."""
    t = workload("tiny")
    assert t.out_fp32 and bench.algorithmic_bytes(t) == 1024 * 1152 + 16 * 1152 + 16 * 2048 + 16 * 4 + 4
    r = workload("ragged")
    L = r.cache_seqlens.astype(np.int64)
    assert L.min() >= 1024 and L.max() <= 65536 and len(L) == 64
    pages = int(((L + 63) // 64).sum())
    assert bench.algorithmic_bytes(r) == int(L.sum()) * 1152 + 64 * 128 * (1152 + 1024 + 4) + 4 * pages


def test_traffic_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    """`traffic` comes from profiles/counters.json only when its source hash is the current one."""
    from mla_decode_attention_paged_amd import profiling
    path = tmp_path / "counters.json"
    path.write_text(json.dumps({"long": {"hbm_bytes_per_launch": 123, "kernel_source_hash": "abc"}}))
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(path))
    monkeypatch.setattr(profiling, "kernel_source_hash", lambda: "abc")
    assert bench.measured_traffic("long") == 123
    assert bench.measured_traffic("ragged") is None
    monkeypatch.setattr(profiling, "kernel_source_hash", lambda: "def")
    assert bench.measured_traffic("long") is None
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("long") is None


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""
