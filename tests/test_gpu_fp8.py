"""FP8 (E4M3) latent cache rows on the HIP path (through the C-ABI) against the fp64 oracle.

The kernel converts the codes to bf16 in registers (K with the exponent of its group scale,
V^T unscaled with each token's power-of-two scale folded into its softmax weight), which is
exact and forms the same products as the bf16 path; so an fp8 cache and a bf16 cache holding
the same values give bit-identical results, and the fp32-output bounds of the bf16 path apply.
"""
import numpy as np
import pytest

from mla_decode_attention_paged_amd import binding as B
from mla_decode_attention_paged_amd import inputs as gen
from mla_decode_attention_paged_amd.device import Runner, to_device
from oracle import mla_oracle as orc
from tests.test_gpu_parity import (F32_LSE_TOL, F32_MAX_TOL, F32_RMSE_TOL, _say, bf16_out_excess, check_dropped_page,
                                   compare, softmax_abs_v)

pytestmark = pytest.mark.gpu

TIGHT = (F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL)


def run(prob, **kw):
    r = Runner(prob, **kw)
    r()
    return r.results()


def oracle(prob, batch_idx=None, causal=False):
    return orc.decode(prob.q, prob.kv_cache, prob.block_table, prob.cache_seqlens, prob.softmax_scale,
                      prob.page_size, batch_indices=batch_idx, causal=causal)


def check(out, lse, ref_o, ref_l, out_fp32, what, wabs=None):
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
    if out_fp32:
        compare(out, lse, ref_o, ref_l, what=what + " fp32", tol=TIGHT)
    else:
        excess = bf16_out_excess(out, ref_o, wabs)
        lerr = float(np.max(np.abs(lse[fin] - ref_l[fin]))) if fin.any() else 0.0
        _say(f"  {what} bf16: max error beyond bf16 rounding {excess:.3e}, lse {lerr:.3e}")
        assert excess <= F32_MAX_TOL and lerr <= F32_LSE_TOL, (what, excess, lerr)


@pytest.mark.parametrize("page", [16, 64])
def test_fp8_gather_bit_exact(page):
    import torch
    prob = gen.make_problem(batch=4, q_len=1, num_heads=16, page_size=page, lengths=[1, 15, page + 1, 700],
                            seed=51, tail="nan", extra_pages=2, kv_format="fp8")
    dev = to_device(prob)
    r = Runner(prob, dev=dev)
    rows = torch.empty((int(prob.cache_seqlens.sum()), 656), dtype=torch.uint8, device="cuda")
    B.mla_debug_gather(r.plan, dev["kv_cache"], dev["block_table"], rows)
    got = rows.cpu().numpy()
    off = 0
    for b in range(prob.batch):
        L = int(prob.cache_seqlens[b])
        assert np.array_equal(got[off:off + L], orc.gather_sequence(prob.kv_cache, prob.block_table[b], L, page))
        off += L


@pytest.mark.parametrize("out_fp32", [True, False])
@pytest.mark.parametrize("page", [16, 48, 64])
def test_fp8_edge_lengths_nan_tails(page, out_fp32):
    lengths = [1, 2, 15, 16, 17, 63, 64, 65, 1000, 5000]
    prob = gen.make_problem(batch=len(lengths), q_len=1, num_heads=16, page_size=page, lengths=lengths, seed=52,
                            tail="nan", extra_pages=3, out_fp32=out_fp32, kv_format="fp8")
    out, lse = run(prob)
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, out_fp32, f"fp8 edges P={page}", None if out_fp32 else softmax_abs_v(prob))


@pytest.mark.parametrize("out_fp32", [True, False])
def test_fp8_many_pieces_per_work_group(out_fp32):
    """Few work-groups, each walking many short FP8 sequences (the three stages reused
    from piece to piece), with empty and one-token sequences among them."""
    rng = np.random.default_rng(53)
    lengths = rng.integers(0, 120, size=300)
    lengths[::13] = 0
    lengths[3::19] = 1
    prob = gen.make_problem(batch=300, q_len=1, num_heads=16, page_size=16, lengths=lengths.tolist(), seed=53,
                            tail="nan", out_fp32=out_fp32, kv_format="fp8")
    r = Runner(prob, num_cus=16)
    assert max(np.diff(r.plan.segments()[1])) > 10
    r()
    out, lse = r.results()
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, out_fp32, "fp8 many pieces", None if out_fp32 else softmax_abs_v(prob))


@pytest.mark.parametrize("heads,q_len", [(16, 2), (32, 1), (64, 1), (128, 1), (48, 1), (128, 2)])
def test_fp8_more_query_rows(heads, q_len):
    prob = gen.make_problem(batch=3, q_len=q_len, num_heads=heads, page_size=64, lengths=[700, 2000, 33], seed=53,
                            out_fp32=True, kv_format="fp8")
    out, lse = run(prob)
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, True, f"fp8 H={heads} S_q={q_len}")


@pytest.mark.parametrize("force", [2, 3, 1000])
def test_fp8_forced_splits(force):
    prob = gen.make_problem(batch=3, q_len=1, num_heads=16, page_size=64, lengths=[4096, 100, 2500], seed=54,
                            out_fp32=True, kv_format="fp8")
    out, lse = run(prob, force_splits=force)
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, True, f"fp8 force={force}")


def test_fp8_causal_two_token():
    prob = gen.make_problem(batch=5, q_len=2, num_heads=16, page_size=16, lengths=[1, 2, 17, 300, 3000], seed=55,
                            tail="nan", extra_pages=1, out_fp32=True, kv_format="fp8")
    out, lse = run(prob, causal=True)
    ref_o, ref_l = oracle(prob, causal=True)
    empty = ~np.isfinite(ref_l)
    assert np.all(out[empty] == 0) and np.all(lse[empty] == -np.inf)
    check(out, lse, ref_o, ref_l, True, "fp8 causal")


def test_fp8_equals_bf16_cache_with_the_same_values():
    """Widening is exact and the arithmetic after it is the bf16 path's: bit-identical."""
    prob = gen.make_problem(batch=4, q_len=1, num_heads=16, page_size=64, lengths=[3000, 64, 5000, 17], seed=56,
                            kv_format="fp8")
    wide = orc.widen_fp8_rows(prob.kv_cache.reshape(-1, 656)).astype(np.float32)
    bits = (wide.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(gen.bf16_bits_to_f32(bits), wide), "widened fp8 values must be exact in bf16"
    prob_bf = gen.Problem(q=prob.q, kv_cache=bits.reshape(prob.kv_cache.shape[0], prob.kv_cache.shape[1], 576),
                          block_table=prob.block_table, cache_seqlens=prob.cache_seqlens,
                          softmax_scale=prob.softmax_scale, page_size=64)
    o8, l8 = run(prob)
    ob, lb = run(prob_bf)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


@pytest.mark.parametrize("name,sample", [("long", [0, 15]), ("paged", [3])])
def test_fp8_full_size_sampled(name, sample):
    _say(f"generating {name} (fp8)")
    prob = gen.make_config(name, kv_format="fp8")
    out, lse = run(prob)
    ref_o, ref_l = oracle(prob, sample)
    compare(out, lse, ref_o, ref_l, batch_idx=sample, what=f"{name} fp8")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_fp8_out_of_range_block_table_entry_drops_its_tokens():
    """A used table entry outside [0, num_pages): its 16-token blocks are masked out (their DMA
    reads page 0), bit 0 of the status word is set, and the rest is exact."""
    prob = gen.make_problem(batch=2, q_len=1, num_heads=16, page_size=64, lengths=[640, 600], seed=31,
                            kv_format="fp8", out_fp32=True)
    bt = prob.block_table.copy()
    bt[1, 3] = prob.num_pages + 5
    bad = gen.Problem(q=prob.q, kv_cache=prob.kv_cache, block_table=bt, cache_seqlens=prob.cache_seqlens,
                      softmax_scale=prob.softmax_scale, page_size=64, out_fp32=True)
    r = Runner(bad)
    r()
    out, lse = r.results()
    assert B.mla_read_status(r.ws) & 1
    ref_o, ref_l = oracle(prob, [0])
    compare(out, lse, ref_o, ref_l, batch_idx=[0], what="fp8 unaffected sequence", tol=TIGHT)
    check_dropped_page(prob, out, lse, seq=1, page_idx=3, tol=TIGHT)
