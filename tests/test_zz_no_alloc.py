"""The entry point that allocates nothing (mla_decode_devplan_noalloc) against the
device-scheduled decode with a caller workspace (mla_decode_devplan), through the C-ABI.

Two calls in a row on one GPU, the second with a smaller problem (the scratch keeps the first
call's contents): each must equal the workspace entry point's result bit for bit (same kernels,
same schedule) and the fp64 oracle within the decode's bounds.  A schedule larger than the
scratch is refused before any launch."""
import numpy as np
import pytest

from mla_decode_attention_paged_amd import binding as B
from mla_decode_attention_paged_amd import inputs as gen
from mla_decode_attention_paged_amd.device import DevplanRunner, problem_struct, to_device
from oracle import mla_oracle as orc
from tests.test_gpu_parity import (F32_LSE_TOL, F32_MAX_TOL, F32_RMSE_TOL, LSE_TOL, MAX_TOL, RMSE_TOL, _say,
                                   compare)

pytestmark = pytest.mark.gpu


def _noalloc(prob, dev, causal=False):
    import torch
    odt = torch.float32 if prob.out_fp32 else torch.bfloat16
    out = torch.full((prob.batch, prob.q_len, prob.num_heads, 512), 5.0, dtype=odt, device="cuda")
    lse = torch.full((prob.batch, prob.q_len, prob.num_heads), 5.0, dtype=torch.float32, device="cuda")
    B.mla_decode_devplan_noalloc(problem_struct(prob, causal), 0, dev["q"], dev["kv_cache"], dev["block_table"],
                                 dev["cache_seqlens"], prob.softmax_scale, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def test_no_alloc_entry_point_matches_the_workspace_entry_point():
    cases = [
        ("ragged batch of 12, 16 heads, bf16",
         gen.make_problem(batch=12, q_len=1, num_heads=16, page_size=64, lengths=None, ragged_range=(1, 20000),
                          seed=71), False),
        ("smaller: 3 sequences, 2 tokens x 64 heads, fp8 rows, fp32 out, causal",
         gen.make_problem(batch=3, q_len=2, num_heads=64, page_size=32, lengths=[900, 1, 2500], seed=72,
                          kv_format="fp8", out_fp32=True, tail="nan", extra_pages=2), True),
    ]
    for what, prob, causal in cases:
        _say(f"  no-alloc call: {what}")
        dev = to_device(prob)
        out, lse = _noalloc(prob, dev, causal)
        r = DevplanRunner(prob, dev=dev, causal=causal)
        r()
        ref_o, ref_l = r.results()
        assert np.array_equal(out, ref_o) and np.array_equal(lse, ref_l), what
        oo, ol = orc.decode(prob.q, prob.kv_cache, prob.block_table, prob.cache_seqlens, prob.softmax_scale,
                            prob.page_size, causal=causal)
        tol = (F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL) if prob.out_fp32 else (RMSE_TOL, MAX_TOL, LSE_TOL)
        compare(out, lse, oo, ol, what=what, tol=tol)      # rows that see no token: out 0, lse -inf on both


def test_no_alloc_refuses_a_schedule_larger_than_its_scratch():
    import torch
    prob = gen.make_problem(batch=2, q_len=1, num_heads=16, page_size=64, lengths=[100, 200], seed=73)
    dev = to_device(prob)
    p = problem_struct(prob)
    out = torch.zeros((2, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
    need = B.devplan_workspace_bytes(p, 1 << 16)
    assert need > (24 << 20)
    with pytest.raises(B.MlaError) as ei:
        B.mla_decode_devplan_noalloc(p, 1 << 16, dev["q"], dev["kv_cache"], dev["block_table"],
                                     dev["cache_seqlens"], prob.softmax_scale, out, None)
    assert ei.value.status == B.MLA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool(torch.all(out == 0))
