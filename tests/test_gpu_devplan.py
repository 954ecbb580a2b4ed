"""Device-scheduled decode (mla_decode_devplan): no host plan; split and merge launches that
take the schedule from the device cache_seqlens.

Checked against the fp64 oracle on the workloads, edge lengths (including empty
contexts and NaN tails), fp8 rows, causal queries, odd worker counts, and with the
device lengths rewritten between calls and between replays of a captured graph.
"""
import numpy as np
import pytest

from mla_decode_attention_paged_amd import inputs as gen
from mla_decode_attention_paged_amd.device import DevplanRunner, to_device
from oracle import mla_oracle as orc
from tests.test_gpu_parity import (F32_LSE_TOL, F32_MAX_TOL, F32_RMSE_TOL, LSE_TOL, MAX_TOL, RMSE_TOL, _say,
                                   bf16_out_excess, compare, compare_every_sequence, softmax_abs_v)

pytestmark = pytest.mark.gpu
TIGHT = (F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL)


def oracle(prob, batch_idx=None, causal=False, seqlens=None):
    sl = prob.cache_seqlens if seqlens is None else seqlens
    return orc.decode(prob.q, prob.kv_cache, prob.block_table, sl, prob.softmax_scale, prob.page_size,
                      batch_indices=batch_idx, causal=causal)


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


def run(prob, **kw):
    r = DevplanRunner(prob, **kw)
    r()
    return r, r.results()


@pytest.mark.parametrize("out_fp32", [True, False])
@pytest.mark.parametrize("kv_format", ["bf16", "fp8"])
def test_devplan_edge_lengths(kv_format, out_fp32):
    lengths = [0, 1, 15, 16, 17, 0, 63, 64, 65, 1000, 5000, 0]
    prob = gen.make_problem(batch=len(lengths), q_len=1, num_heads=16, page_size=16, lengths=lengths, seed=61,
                            tail="nan", extra_pages=2, out_fp32=out_fp32, kv_format=kv_format)
    _, (out, lse) = run(prob)
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, out_fp32, f"devplan edges {kv_format}", None if out_fp32 else softmax_abs_v(prob))


@pytest.mark.parametrize("workers", [1, 3, 7, 64, 300])
def test_devplan_worker_counts(workers):
    """Few and many work-groups, including more work-groups than blocks (empty ranges)."""
    prob = gen.make_problem(batch=4, q_len=1, num_heads=16, page_size=64, lengths=[3000, 20, 700, 64], seed=62,
                            out_fp32=True)
    _, (out, lse) = run(prob, num_workers=workers)
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, True, f"devplan W={workers}")


@pytest.mark.parametrize("heads,q_len,causal", [(16, 2, False), (16, 2, True), (32, 1, False), (64, 1, False),
                                                (128, 1, False), (48, 1, False), (8, 2, True), (128, 2, True)])
def test_devplan_more_rows(heads, q_len, causal):
    prob = gen.make_problem(batch=3, q_len=q_len, num_heads=heads, page_size=64, lengths=[700, 2000, 33], seed=63,
                            out_fp32=True)
    _, (out, lse) = run(prob, causal=causal)
    ref_o, ref_l = oracle(prob, causal=causal)
    check(out, lse, ref_o, ref_l, True, f"devplan H={heads} S_q={q_len} causal={causal}")


def test_devplan_lengths_change_between_calls_and_graph_replays():
    import torch
    rng = np.random.default_rng(64)
    # every sequence has pages mapped for 4096 tokens; the calls use shorter, changing lengths
    prob = gen.make_problem(batch=6, q_len=1, num_heads=16, page_size=64, lengths=[4096] * 6, seed=64,
                            out_fp32=True)
    cap = prob.max_pages_per_seq * prob.page_size
    r = DevplanRunner(prob)
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


def test_devplan_repeated_calls_bit_identical():
    prob = gen.make_problem(batch=4, q_len=1, num_heads=16, page_size=64, lengths=[9000, 100, 5000, 64], seed=65)
    r, (o1, l1) = run(prob)
    for _ in range(3):
        r()
        o2, l2 = r.results()
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name", ["tiny", "paged", "two_token", "long", "ragged"])
def test_devplan_workloads(name):
    _say(f"generating {name}")
    prob = gen.make_config(name)
    _, (out, lse) = run(prob)
    _say(f"oracle on all {prob.batch} sequences")
    ref_o, ref_l = oracle(prob)
    tol = TIGHT if prob.out_fp32 else (RMSE_TOL, MAX_TOL, LSE_TOL)
    compare_every_sequence(out, lse, ref_o, ref_l, f"devplan {name}", tol=tol)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_devplan_cache_beyond_4gib(kv):
    """The device schedule on a cache larger than 4 GiB with pages past the 4-GiB offset:
    bit-identical to the same problem on a compact cache, and within the fp32 bounds of
    the oracle."""
    import torch
    from tests.test_gpu_parity import _spread_beyond_4gib
    prob = gen.make_problem(batch=3, q_len=1, num_heads=16, page_size=64, lengths=[3000, 700, 65], seed=29,
                            out_fp32=True, kv_format=kv)
    big_pages = 65536 if kv == "bf16" else 110000
    _say(f"  devplan cache beyond 4 GiB: kv={kv} pages={big_pages}")
    big_prob, dev = _spread_beyond_4gib(prob, big_pages, seed=29)
    r_big, (out_b, lse_b) = run(big_prob, dev=dev)
    r_small, (out_s, lse_s) = run(prob)
    assert np.array_equal(out_b, out_s) and np.array_equal(lse_b, lse_s)
    ref_o, ref_l = oracle(prob)
    check(out_b, lse_b, ref_o, ref_l, True, f"devplan beyond 4 GiB {kv}")
    del r_big, dev
    torch.cuda.empty_cache()
