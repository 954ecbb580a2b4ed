"""Causal multi-token queries on the HIP path (through the C-ABI) against the fp64 oracle.

Query token i of S_q sees the first L - (S_q - 1 - i) cached tokens.  Rows that see
no token (L < S_q - i) must come back as out = 0, lse = -inf; split sequences whose
last piece a row cannot see exercise -inf partials in the merge.
"""
import numpy as np
import pytest

from mla_decode_attention_paged_amd import inputs as gen
from mla_decode_attention_paged_amd.device import Runner
from oracle import mla_oracle as orc
from tests.test_gpu_parity import (F32_LSE_TOL, F32_MAX_TOL, F32_RMSE_TOL, LSE_TOL, MAX_TOL, RMSE_TOL, _say,
                                   bf16_out_excess, compare, compare_every_sequence, softmax_abs_v)

pytestmark = pytest.mark.gpu

EDGE_LENGTHS = [1, 2, 3, 7, 15, 16, 17, 18, 33, 1000, 4096]


def run(prob, **kw):
    r = Runner(prob, causal=True, **kw)
    r()
    return r.results()


def oracle(prob, batch_idx=None):
    return orc.decode(prob.q, prob.kv_cache, prob.block_table, prob.cache_seqlens, prob.softmax_scale,
                      prob.page_size, batch_indices=batch_idx, causal=True)


def check(out, lse, ref_o, ref_l, out_fp32, what, wabs=None):
    assert np.array_equal(np.isfinite(lse), np.isfinite(ref_l)), f"{what}: lse finiteness differs"
    empty = ~np.isfinite(ref_l)
    assert np.all(lse[empty] == -np.inf) and np.all(out[empty] == 0), f"{what}: empty rows"
    if out_fp32:
        compare(out, lse, ref_o, ref_l, what=what + " fp32", tol=(F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL))
    else:
        excess = bf16_out_excess(out, ref_o, wabs)
        lerr = float(np.max(np.abs(lse[~empty] - ref_l[~empty])))
        _say(f"  {what} bf16: max error beyond bf16 rounding {excess:.3e}, lse {lerr:.3e}")
        assert excess <= F32_MAX_TOL and lerr <= F32_LSE_TOL, (what, excess, lerr)


@pytest.mark.parametrize("heads,q_len", [(8, 2), (16, 2), (16, 3), (32, 2), (64, 2), (16, 8), (128, 2)])
@pytest.mark.parametrize("out_fp32", [True, False])
def test_causal_edge_lengths(heads, q_len, out_fp32):
    prob = gen.make_problem(batch=len(EDGE_LENGTHS), q_len=q_len, num_heads=heads, page_size=16,
                            lengths=EDGE_LENGTHS, seed=21, tail="nan", extra_pages=2, out_fp32=out_fp32)
    out, lse = run(prob)
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, out_fp32, f"causal H={heads} S_q={q_len}",
          None if out_fp32 else softmax_abs_v(prob, causal=True))


@pytest.mark.parametrize("heads,q_len,rpg", [(16, 2, 32), (8, 4, 32), (16, 4, 64), (32, 2, 16), (16, 8, 16),
                                          (64, 2, 128), (128, 2, 128), (32, 4, 128),
                                          (128, 2, 64)])
@pytest.mark.parametrize("out_fp32", [True, False])
def test_causal_rows_per_group(heads, q_len, rpg, out_fp32):
    """The causal limit in every kernel layout asked for explicitly: the 32-row kernel, the wide
    kernel with 64 rows (two waves per 32 rows) and 128, and the 16-row kernel where the default
    would be a wider one."""
    prob = gen.make_problem(batch=len(EDGE_LENGTHS), q_len=q_len, num_heads=heads, page_size=16,
                            lengths=EDGE_LENGTHS, seed=24, tail="nan", extra_pages=2, out_fp32=out_fp32)
    r = Runner(prob, causal=True, rows_per_group=rpg)
    assert r.plan.info()["rows_per_group"] == rpg
    r()
    out, lse = r.results()
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, out_fp32, f"causal H={heads} S_q={q_len} rpg={rpg}",
          None if out_fp32 else softmax_abs_v(prob, causal=True))


@pytest.mark.parametrize("heads,q_len", [(8, 2), (16, 2), (64, 2)])
@pytest.mark.parametrize("force", [2, 3, 1000])
def test_causal_forced_splits(heads, q_len, force):
    """Pieces that end before a row's last visible token, or start after it (-inf partials)."""
    prob = gen.make_problem(batch=4, q_len=q_len, num_heads=heads, page_size=64, lengths=[17, 33, 100, 2500],
                            seed=22, out_fp32=True)
    out, lse = run(prob, force_splits=force)
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, True, f"causal force={force} H={heads}")


def test_causal_last_token_matches_unmasked_call():
    """The last query token sees every cached token: bit-identical to the unmasked call's row."""
    prob = gen.make_problem(batch=3, q_len=2, num_heads=16, page_size=64, lengths=[1500, 300, 16], seed=23,
                            out_fp32=True)
    oc, lc = run(prob)
    r = Runner(prob)
    r()
    o, l = r.results()
    assert np.array_equal(oc[:, 1], o[:, 1]) and np.array_equal(lc[:, 1], l[:, 1])
    assert np.max(np.abs(oc[:, 0] - o[:, 0])) > 1e-4, "the mask changed nothing for token 0"


def test_causal_two_token_full_size():
    _say("generating two_token")
    prob = gen.make_config("two_token")
    out, lse = run(prob)
    _say(f"oracle on all {prob.batch} sequences")
    ref_o, ref_l = oracle(prob)
    compare_every_sequence(out, lse, ref_o, ref_l, "two_token causal")
