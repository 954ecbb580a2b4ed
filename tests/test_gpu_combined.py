"""One-launch decode: the 16-row split kernel combines split sequences itself.

Host plan (mla_decode_stages with MLA_STAGE_COMBINED) and device schedule
(mla_decode_devplan_combined), each checked against the fp64 oracle and against its
two-launch counterpart (same partial results; only the order of the combine's additions
differs, so fp32 outputs agree within a few ulps).  The election counter must be back at zero
after every launch: repeated calls, calls with other stages in between and graph replays all
give the same results.
"""
import numpy as np
import pytest

from mla_decode_attention_paged_amd import binding as B
from mla_decode_attention_paged_amd import inputs as gen
from mla_decode_attention_paged_amd.device import DevplanRunner, Runner
from oracle import mla_oracle as orc
from tests.test_gpu_parity import (F32_LSE_TOL, F32_MAX_TOL, F32_RMSE_TOL, LSE_TOL, MAX_TOL, RMSE_TOL, _say,
                                   bf16_out_excess, compare, compare_every_sequence, softmax_abs_v)

pytestmark = pytest.mark.gpu
TIGHT = (F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL)


def oracle(prob, causal=False, seqlens=None):
    sl = prob.cache_seqlens if seqlens is None else seqlens
    return orc.decode(prob.q, prob.kv_cache, prob.block_table, sl, prob.softmax_scale, prob.page_size, causal=causal)


def check(out, lse, ref_o, ref_l, out_fp32, what, wabs=None):
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
    assert np.all(out[~fin] == 0), f"{what}: empty rows not zero"
    if out_fp32:
        compare(out, lse, ref_o, ref_l, what=what + " fp32", tol=TIGHT)
    else:
        excess = bf16_out_excess(out, ref_o, wabs)
        lerr = float(np.max(np.abs(lse[fin] - ref_l[fin]))) if fin.any() else 0.0
        _say(f"  {what} bf16: max error beyond bf16 rounding {excess:.3e}, lse {lerr:.3e}")
        assert excess <= F32_MAX_TOL and lerr <= F32_LSE_TOL, (what, excess, lerr)


def close_to_two_launch(o1, l1, o2, l2, out_fp32, what):
    """The combined and the two-launch results: same partials, different summation order."""
    fin = np.isfinite(l2)
    assert np.array_equal(np.isfinite(l1), fin), what
    assert np.max(np.abs(l1[fin] - l2[fin]), initial=0.0) <= 8e-6, what
    scale = np.max(np.abs(o2), initial=1.0)
    tol = 1e-6 if out_fp32 else 2 ** -7        # bf16 output: one rounding step either way
    assert np.max(np.abs(o1 - o2)) <= tol * scale, (what, float(np.max(np.abs(o1 - o2))))


def host_pair(prob, **kw):
    r = Runner(prob, **kw)
    assert r.plan.info()["rows_per_group"] == 16
    r(stages=B.MLA_STAGE_COMBINED)
    oc, lc = r.results()
    r()
    o2, l2 = r.results()
    return r, (oc, lc), (o2, l2)


@pytest.mark.parametrize("out_fp32", [True, False])
@pytest.mark.parametrize("kv_format", ["bf16", "fp8"])
def test_combined_host_edge_lengths(kv_format, out_fp32):
    lengths = [0, 1, 15, 16, 17, 0, 63, 64, 65, 1000, 5000, 0, 12000]
    prob = gen.make_problem(batch=len(lengths), q_len=1, num_heads=16, page_size=16, lengths=lengths, seed=81,
                            tail="nan", extra_pages=2, out_fp32=out_fp32, kv_format=kv_format)
    r, (oc, lc), (o2, l2) = host_pair(prob, num_cus=64)
    assert r.plan.info()["num_combine"] > 0
    ref_o, ref_l = oracle(prob)
    check(oc, lc, ref_o, ref_l, out_fp32, f"combined {kv_format}", None if out_fp32 else softmax_abs_v(prob))
    close_to_two_launch(oc, lc, o2, l2, out_fp32, f"combined vs two launches {kv_format}")


@pytest.mark.parametrize("force", [2, 3, 17, 1000])
def test_combined_host_forced_splits(force):
    """Every sequence cut into `force` pieces (1000: one piece per 16-token block), more
    pieces than one combine batch."""
    prob = gen.make_problem(batch=3, q_len=1, num_heads=16, page_size=64, lengths=[4096, 100, 2500], seed=82,
                            out_fp32=True)
    r, (oc, lc), (o2, l2) = host_pair(prob, force_splits=force)
    ref_o, ref_l = oracle(prob)
    check(oc, lc, ref_o, ref_l, True, f"combined force={force}")
    close_to_two_launch(oc, lc, o2, l2, True, f"combined vs two launches force={force}")


@pytest.mark.parametrize("heads,q_len,causal", [(16, 2, False), (16, 2, True), (32, 1, False), (48, 1, False)])
def test_combined_host_row_groups(heads, q_len, causal):
    """Several 16-row groups: one counter per (sequence, row group)."""
    prob = gen.make_problem(batch=3, q_len=q_len, num_heads=heads, page_size=64, lengths=[700, 9000, 33], seed=83,
                            out_fp32=True)
    r, (oc, lc), (o2, l2) = host_pair(prob, causal=causal, rows_per_group=16, num_cus=96)
    assert r.plan.info()["row_groups"] == heads * q_len // 16
    ref_o, ref_l = oracle(prob, causal=causal)
    check(oc, lc, ref_o, ref_l, True, f"combined H={heads} S_q={q_len} causal={causal}")
    close_to_two_launch(oc, lc, o2, l2, True, "combined vs two launches (row groups)")


def test_combined_host_counters_return_to_zero():
    """Combined calls repeated, interleaved with two-launch calls and split-only calls: every
    combined call gives the same bits (a counter left non-zero would change the election)."""
    prob = gen.make_problem(batch=5, q_len=1, num_heads=16, page_size=64, lengths=[9000, 100, 5000, 64, 3000],
                            seed=84)
    r = Runner(prob, num_cus=40)
    r(stages=B.MLA_STAGE_COMBINED)
    o1, l1 = r.results()
    for stages in (B.MLA_STAGE_COMBINED, B.MLA_STAGE_ALL, B.MLA_STAGE_SPLIT, B.MLA_STAGE_COMBINED,
                   B.MLA_STAGE_COMBINED):
        r(stages=stages)
        if stages == B.MLA_STAGE_COMBINED:
            o2, l2 = r.results()
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_combined_host_graph_replays():
    import torch
    prob = gen.make_problem(batch=4, q_len=1, num_heads=16, page_size=64, lengths=[6000, 300, 2048, 4000], seed=85,
                            out_fp32=True)
    r = Runner(prob, num_cus=64)
    r(stages=B.MLA_STAGE_COMBINED)
    ref, ref_l = r.results()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            r(stream=side, stages=B.MLA_STAGE_COMBINED)
    torch.cuda.current_stream().wait_stream(side)
    for i in range(4):
        r.out.zero_()
        r()                                   # eager two-launch work between the replays
        r.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        o, l = r.results()
        assert np.array_equal(o, ref) and np.array_equal(l, ref_l), f"replay {i}"


@pytest.mark.parametrize("name", ["paged", "long"])
def test_combined_host_full_size(name):
    _say(f"generating {name}")
    prob = gen.make_config(name)
    r, (oc, lc), (o2, l2) = host_pair(prob)
    _say(f"oracle on all {prob.batch} sequences")
    ref_o, ref_l = oracle(prob)
    tol = TIGHT if prob.out_fp32 else (RMSE_TOL, MAX_TOL, LSE_TOL)
    compare_every_sequence(oc, lc, ref_o, ref_l, f"combined {name}", tol=tol)
    close_to_two_launch(oc, lc, o2, l2, prob.out_fp32, f"combined vs two launches {name}")


# ---- device schedule

@pytest.mark.parametrize("out_fp32", [True, False])
@pytest.mark.parametrize("kv_format", ["bf16", "fp8"])
def test_combined_devplan_edge_lengths(kv_format, out_fp32):
    lengths = [0, 1, 15, 16, 17, 0, 63, 64, 65, 1000, 5000, 0]
    prob = gen.make_problem(batch=len(lengths), q_len=1, num_heads=16, page_size=16, lengths=lengths, seed=86,
                            tail="nan", extra_pages=2, out_fp32=out_fp32, kv_format=kv_format)
    rc = DevplanRunner(prob, combined=True)
    rc()
    oc, lc = rc.results()
    r2 = DevplanRunner(prob, dev=rc.dev)
    r2()
    o2, l2 = r2.results()
    ref_o, ref_l = oracle(prob)
    check(oc, lc, ref_o, ref_l, out_fp32, f"devplan combined {kv_format}", None if out_fp32 else softmax_abs_v(prob))
    close_to_two_launch(oc, lc, o2, l2, out_fp32, f"devplan combined vs two launches {kv_format}")


@pytest.mark.parametrize("workers", [1, 3, 7, 64, 300])
def test_combined_devplan_worker_counts(workers):
    prob = gen.make_problem(batch=4, q_len=1, num_heads=16, page_size=64, lengths=[3000, 20, 700, 64], seed=87,
                            out_fp32=True)
    r = DevplanRunner(prob, num_workers=workers, combined=True)
    r()
    o, l = r.results()
    ref_o, ref_l = oracle(prob)
    check(o, l, ref_o, ref_l, True, f"devplan combined W={workers}")


@pytest.mark.parametrize("heads,q_len,causal", [(16, 2, True), (32, 1, False), (128, 1, False)])
def test_combined_devplan_more_rows(heads, q_len, causal):
    prob = gen.make_problem(batch=3, q_len=q_len, num_heads=heads, page_size=64, lengths=[700, 2000, 33], seed=88,
                            out_fp32=True)
    r = DevplanRunner(prob, causal=causal, combined=True)
    r()
    o, l = r.results()
    ref_o, ref_l = oracle(prob, causal=causal)
    check(o, l, ref_o, ref_l, True, f"devplan combined H={heads} S_q={q_len} causal={causal}")


def test_combined_devplan_lengths_change_between_calls_and_graph_replays():
    import torch
    rng = np.random.default_rng(89)
    prob = gen.make_problem(batch=6, q_len=1, num_heads=16, page_size=64, lengths=[4096] * 6, seed=89,
                            out_fp32=True)
    cap = prob.max_pages_per_seq * prob.page_size
    r = DevplanRunner(prob, combined=True)
    sl_dev = r.dev["cache_seqlens"]
    trials = [np.array([4096, 300, 2048, 64, 1, 3000], dtype=np.int32)] + \
        [rng.integers(0, cap, size=6, endpoint=True).astype(np.int32) for _ in range(3)]
    trials[2][4] = 0
    for i, sl in enumerate(trials):
        sl = np.minimum(sl, cap).astype(np.int32)
        sl_dev.copy_(torch.from_numpy(sl))
        r()
        o, l = r.results()
        ref_o, ref_l = oracle(prob, seqlens=sl)
        check(o, l, ref_o, ref_l, True, f"eager call {i} lengths {sl.tolist()}")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            r(stream=side)
    torch.cuda.current_stream().wait_stream(side)
    for i, sl in enumerate(reversed(trials)):
        sl = np.minimum(sl, cap).astype(np.int32)
        sl_dev.copy_(torch.from_numpy(sl))
        r.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        o, l = r.results()
        ref_o, ref_l = oracle(prob, seqlens=sl)
        check(o, l, ref_o, ref_l, True, f"replay {i} lengths {sl.tolist()}")


@pytest.mark.parametrize("name", ["paged", "long", "two_token"])
def test_combined_devplan_workloads(name):
    _say(f"generating {name}")
    prob = gen.make_config(name)
    r = DevplanRunner(prob, combined=True)
    r()
    out, lse = r.results()
    _say(f"oracle on all {prob.batch} sequences")
    ref_o, ref_l = oracle(prob)
    tol = TIGHT if prob.out_fp32 else (RMSE_TOL, MAX_TOL, LSE_TOL)
    compare_every_sequence(out, lse, ref_o, ref_l, f"devplan combined {name}", tol=tol)
