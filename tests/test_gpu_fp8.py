"""FP8 (E4M3) latent cache rows on the HIP path (through the C-ABI) against the fp64 oracle.

The 16-row kernel converts the codes to bf16 in registers (K with the exponent of its group
scale, V^T unscaled with each token's power-of-two scale folded into its softmax weight); the
128-row kernel converts each block once in LDS into the bf16 layout (code times the scale's
power of two).  Both are exact and form the same products as the bf16 path of the same kernel;
so an fp8 cache and a bf16 cache holding the same values give bit-identical results, and the
fp32-output bounds of the bf16 path apply.  Tests with 128 heads run the 128-row kernel (the
default when R is a multiple of 128).
"""
import numpy as np
import pytest

from mla_decode_attention_paged_amd import binding as B
from mla_decode_attention_paged_amd import inputs as gen
from mla_decode_attention_paged_amd.device import Runner, to_device
from oracle import mla_oracle as orc
from tests.test_gpu_parity import (F32_LSE_TOL, F32_MAX_TOL, F32_RMSE_TOL, _say, bf16_out_excess, check_dropped_page,
                                   compare, compare_every_sequence, softmax_abs_v)

pytestmark = pytest.mark.gpu

TIGHT = (F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL)


def run(prob, **kw):
    r = Runner(prob, **kw)
    r()
    return r.results()


def oracle(prob, batch_idx=None, causal=False):
    return orc.decode(prob.q, prob.kv_cache, prob.block_table, prob.cache_seqlens, prob.softmax_scale,
                      prob.page_size, batch_indices=batch_idx, causal=causal)


def with_page_zero_unmapped(prob):
    """The same problem with physical page 0 swapped with an unmapped page and its latent codes
    set to NaN (0x7F): the page a DMA reads for an out-of-range table entry then holds NaN."""
    bt = prob.block_table.copy()
    used = set(bt[bt >= 0].tolist())
    u = next(p for p in range(prob.num_pages) if p not in used)
    kv = prob.kv_cache.copy()
    kv[[0, u]] = kv[[u, 0]]
    bt[bt == 0] = u
    kv[0, :, :512] = 0x7F
    return gen.Problem(q=prob.q, kv_cache=kv, block_table=bt, cache_seqlens=prob.cache_seqlens,
                       softmax_scale=prob.softmax_scale, page_size=prob.page_size, out_fp32=prob.out_fp32)


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


@pytest.mark.parametrize("heads", [16, 128])
@pytest.mark.parametrize("out_fp32", [True, False])
@pytest.mark.parametrize("page", [16, 48, 64])
def test_fp8_edge_lengths_nan_tails(page, out_fp32, heads):
    lengths = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 1000, 5000]
    prob = gen.make_problem(batch=len(lengths), q_len=1, num_heads=heads, page_size=page, lengths=lengths, seed=52,
                            tail="nan", extra_pages=3, out_fp32=out_fp32, kv_format="fp8")
    r = Runner(prob)
    assert r.plan.info()["rows_per_group"] == (128 if heads == 128 else 16)
    r()
    out, lse = r.results()
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, out_fp32, f"fp8 edges P={page} H={heads}", None if out_fp32 else softmax_abs_v(prob))


@pytest.mark.parametrize("heads", [16, 128])
@pytest.mark.parametrize("out_fp32", [True, False])
def test_fp8_many_pieces_per_work_group(out_fp32, heads):
    """Few work-groups, each walking many short FP8 sequences (the stages or slots reused
    from piece to piece), with empty and one-token sequences among them."""
    rng = np.random.default_rng(53)
    lengths = rng.integers(0, 120, size=300)
    lengths[::13] = 0
    lengths[3::19] = 1
    prob = gen.make_problem(batch=300, q_len=1, num_heads=heads, page_size=16, lengths=lengths.tolist(), seed=53,
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


@pytest.mark.parametrize("heads", [16, 128])
@pytest.mark.parametrize("force", [2, 3, 1000])
def test_fp8_forced_splits(force, heads):
    prob = gen.make_problem(batch=3, q_len=1, num_heads=heads, page_size=64, lengths=[4096, 100, 2500], seed=54,
                            out_fp32=True, kv_format="fp8")
    out, lse = run(prob, force_splits=force)
    ref_o, ref_l = oracle(prob)
    check(out, lse, ref_o, ref_l, True, f"fp8 force={force} H={heads}")


@pytest.mark.parametrize("heads", [16, 32, 64])
def test_fp8_causal_two_token(heads):
    prob = gen.make_problem(batch=5, q_len=2, num_heads=heads, page_size=16, lengths=[1, 2, 17, 300, 3000], seed=55,
                            tail="nan", extra_pages=1, out_fp32=True, kv_format="fp8")
    out, lse = run(prob, causal=True)
    ref_o, ref_l = oracle(prob, causal=True)
    empty = ~np.isfinite(ref_l)
    assert np.all(out[empty] == 0) and np.all(lse[empty] == -np.inf)
    check(out, lse, ref_o, ref_l, True, "fp8 causal")


@pytest.mark.parametrize("heads", [16, 128])
def test_fp8_equals_bf16_cache_with_the_same_values(heads):
    """Widening is exact and the arithmetic after it is the bf16 path's: bit-identical."""
    prob = gen.make_problem(batch=4, q_len=1, num_heads=heads, page_size=64, lengths=[3000, 64, 5000, 17], seed=56,
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


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["paged", "two_token", "long", "ragged"])
def test_fp8_full_size(name):
    _say(f"generating {name} (fp8)")
    prob = gen.make_config(name, kv_format="fp8")
    out, lse = run(prob)
    _say(f"oracle on all {prob.batch} sequences")
    ref_o, ref_l = oracle(prob)
    compare_every_sequence(out, lse, ref_o, ref_l, f"{name} fp8")


@pytest.mark.parametrize("heads", [64, 128])
@pytest.mark.parametrize("out_fp32", [True, False])
def test_fp8_scales_with_mantissa_bits_use_the_exponent_only(out_fp32, heads):
    """Group scales that are not powers of two (1.5 * 2^e, 1.9375 * 2^e): only their exponent
    counts (the row format; the oracle decodes it that way).  Equal, bit for bit, to the same
    cache with the scales' mantissas cleared, and to the oracle within the usual bounds."""
    prob = gen.make_problem(batch=3, q_len=1, num_heads=heads, page_size=64, lengths=[2100, 333, 64], seed=57,
                            kv_format="fp8", out_fp32=out_fp32)
    kv = prob.kv_cache.copy()
    sc = np.ascontiguousarray(kv[..., 640:656]).view(np.uint32)
    mant = np.where(np.arange(sc.size).reshape(sc.shape) % 2 == 0, 0x00400000, 0x00780000).astype(np.uint32)
    kv[..., 640:656] = (sc | mant).view(np.uint8)
    odd = gen.Problem(q=prob.q, kv_cache=kv, block_table=prob.block_table, cache_seqlens=prob.cache_seqlens,
                      softmax_scale=prob.softmax_scale, page_size=64, out_fp32=out_fp32)
    o1, l1 = run(odd)
    o0, l0 = run(prob)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)
    ref_o, ref_l = oracle(odd)
    check(o1, l1, ref_o, ref_l, out_fp32, "scales with mantissa bits", None if out_fp32 else softmax_abs_v(odd))


@pytest.mark.parametrize("heads", [16, 128])
def test_fp8_out_of_range_block_table_entry_drops_its_tokens(heads):
    """A used table entry outside [0, num_pages): its tokens are masked out (their DMA reads
    page 0), bit 0 of the status word is set, and the rest is exact."""
    prob = with_page_zero_unmapped(gen.make_problem(batch=2, q_len=1, num_heads=heads, page_size=64,
                                                    lengths=[640, 600], seed=31, extra_pages=1, kv_format="fp8",
                                                    out_fp32=True))
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


@pytest.mark.parametrize("out_fp32", [True, False])
@pytest.mark.parametrize("heads,q_len", [(128, 1), (64, 1), (32, 2)])
def test_fp8_wide_and_16_row_kernels_agree(out_fp32, heads, q_len):
    """The wide kernel (the default at 128 and 64 rows) against the 16-row kernel forced on the
    same FP8 problem: both within the oracle's bounds, and their lse within 1e-5 of each other
    (the two sum the same products in different orders)."""
    prob = gen.make_problem(batch=4, q_len=q_len, num_heads=heads, page_size=64, lengths=[4000, 1, 700, 2049],
                            seed=58, out_fp32=out_fp32, kv_format="fp8")
    rw = Runner(prob)
    r16 = Runner(prob, rows_per_group=16)
    R = heads * q_len
    assert rw.plan.info()["rows_per_group"] == R and r16.plan.info()["rows_per_group"] == 16
    rw()
    r16()
    ow, lw = rw.results()
    o16, l16 = r16.results()
    ref_o, ref_l = oracle(prob)
    wabs = None if out_fp32 else softmax_abs_v(prob)
    check(ow, lw, ref_o, ref_l, out_fp32, f"fp8 {R} rows", wabs)
    check(o16, l16, ref_o, ref_l, out_fp32, "fp8 16 rows", wabs)
    assert np.max(np.abs(lw - l16)) <= 1e-5


def test_fp8_wide_dropped_half_block():
    """Page size 16 at 128 heads: an out-of-range entry drops one 16-token half of a 32-token block
    of the 128-row kernel (the first half in sequence 0, the second in sequence 1); page 0, which
    the DMA reads instead, holds NaN codes.  The status bit is set and the rest is exact."""
    prob = with_page_zero_unmapped(gen.make_problem(batch=2, q_len=1, num_heads=128, page_size=16,
                                                    lengths=[640, 650], seed=59, tail="nan", extra_pages=2,
                                                    out_fp32=True, kv_format="fp8"))
    bt = prob.block_table.copy()
    bt[0, 10] = -1
    bt[1, 5] = prob.num_pages + 3
    bad = gen.Problem(q=prob.q, kv_cache=prob.kv_cache, block_table=bt, cache_seqlens=prob.cache_seqlens,
                      softmax_scale=prob.softmax_scale, page_size=16, out_fp32=True)
    r = Runner(bad)
    assert r.plan.info()["rows_per_group"] == 128
    r()
    out, lse = r.results()
    assert B.mla_read_status(r.ws) & 1
    check_dropped_page(prob, out, lse, seq=0, page_idx=10, tol=TIGHT)
    check_dropped_page(prob, out, lse, seq=1, page_idx=5, tol=TIGHT)
