"""HIP path (through the C-ABI) against the fp64 oracle.  Needs an MI355X.

Tolerances (pooled over all compared elements of a call):
  out: RMSE <= 1e-3 and max |err| <= 1e-2;   lse: max |err| <= 1e-3.
The bf16 output rounding alone contributes about 2e-4 RMSE / 2e-3 max on
N(0,1) inputs; bf16 P in the PV product adds a little more.
"""
import sys

import numpy as np
import pytest

from mla_decode_attention_paged_amd import binding as B
from mla_decode_attention_paged_amd import inputs as gen
from mla_decode_attention_paged_amd.device import Runner, to_device
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

RMSE_TOL, MAX_TOL, LSE_TOL = 1e-3, 1e-2, 1e-3
# fp32 output: the kernel keeps ~16-bit weights (bf16 hi + lo) and fp32 sums
F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL = 1e-5, 1e-4, 1e-5


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place at |x| (the most round-to-nearest can move x)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


# bf16 output: the kernel rounds each softmax weight to bf16 (relative error <= 2^-8) before
# O += V^T P^T, so on top of the output's own rounding an element may move by up to
# 2^-8 sum_t p_t |v_t| / sum_t p_t.
P_BF16_REL = 2.0 ** -8


def softmax_abs_v(prob, batch_idx=None, causal=False, seqlens=None):
    """sum_t p_t |v_t| / sum_t p_t per output element: the oracle's softmax weights (same
    gather, same causal limits) applied to |V|."""
    B, s_q, h = prob.q.shape[:3]
    sl = prob.cache_seqlens if seqlens is None else seqlens
    res = np.zeros((B, s_q, h, orc.D_V))
    for b in (range(B) if batch_idx is None else batch_idx):
        k = orc.widen_rows(orc.gather_sequence(prob.kv_cache, prob.block_table[b], int(sl[b]), prob.page_size))
        for i in range(s_q):
            vis = max(0, int(sl[b]) - s_q + i + 1) if causal else int(sl[b])
            res[b, i], _ = orc.attend(orc.widen_bf16(prob.q[b, i]), k[:vis], np.abs(k[:vis, :orc.D_V]),
                                      prob.softmax_scale)
    return res


def bf16_out_excess(out, ref_o, wabs):
    """Largest error of a bf16 output beyond its own rounding and the bf16-weight bound."""
    return float(np.max(np.abs(out - ref_o) - bf16_half_ulp(ref_o) - P_BF16_REL * wabs))


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def fp32_ulp(x):
    """One float32 unit in the last place at |x|."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 23)


def compare(out, lse, ref_out, ref_lse, batch_idx=None, what="", tol=(RMSE_TOL, MAX_TOL, LSE_TOL), lse_ulps=0):
    """Pooled RMSE and max |err| of out, max |err| of the finite lse values; lse_ulps > 0 also
    allows that many float32 units of |lse| (an fp32 lse near 100 cannot be closer than
    about 8e-6 to the exact value)."""
    if batch_idx is not None:
        out, lse, ref_out, ref_lse = out[batch_idx], lse[batch_idx], ref_out[batch_idx], ref_lse[batch_idx]
    err = out - ref_out
    rmse = float(np.sqrt(np.mean(err ** 2)))
    mx = float(np.max(np.abs(err)))
    finite = np.isfinite(ref_lse)
    lerr = float(np.max(np.abs(lse[finite] - ref_lse[finite]) - lse_ulps * fp32_ulp(ref_lse[finite]))) \
        if finite.any() else 0.0
    assert np.array_equal(np.isfinite(lse), finite), f"{what}: lse finiteness differs"
    _say(f"  {what}: rmse {rmse:.3e} max {mx:.3e} lse {lerr:.3e}")
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    assert rmse <= tol[0] and mx <= tol[1] and lerr <= tol[2], (what, rmse, mx, lerr)
    return rmse, mx, lerr


def check_short_contexts(out, lse, ref_o, ref_l, out_fp32, what, wabs=None, lse_ulps=0):
    """Contexts of a few tokens give |out| up to ~4, where bf16 output rounding alone moves a
    value by up to 2^-7 (more than the pooled max-abs bound for long N(0,1) contexts).  fp32
    output is held to the fp32-path bounds; bf16 output to its rounding, the bf16-weight bound
    (wabs = softmax_abs_v) and the fp32-path bound."""
    if out_fp32:
        compare(out, lse, ref_o, ref_l, what=what + " fp32", tol=(F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL),
                lse_ulps=lse_ulps)
    else:
        excess = bf16_out_excess(out, ref_o, wabs)
        _say(f"  {what} bf16: max error beyond bf16 rounding {excess:.3e}")
        assert excess <= F32_MAX_TOL, (what, excess)
        fin = np.isfinite(ref_l)                      # L = 0 rows: lse = -inf on both sides
        assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
        assert np.array_equal(lse[~fin], ref_l[~fin]), f"{what}: non-finite lse differs"
        if fin.any():
            assert np.max(np.abs(lse[fin] - ref_l[fin]) - lse_ulps * fp32_ulp(ref_l[fin])) <= F32_LSE_TOL, what


def run(prob, **kw):
    r = Runner(prob, **kw)
    r()
    return r.results()


def oracle(prob, batch_idx=None):
    return orc.decode(prob.q, prob.kv_cache, prob.block_table, prob.cache_seqlens, prob.softmax_scale,
                      prob.page_size, batch_indices=batch_idx)


# ----------------------------------------------------------------------------- gather
@pytest.mark.parametrize("page", [16, 64, 1024])
def test_gather_bit_exact(page):
    import torch
    prob = gen.make_problem(batch=5, q_len=1, num_heads=16, page_size=page, lengths=[1, 15, page, page + 1, 3000],
                            seed=3, tail="nan", extra_pages=2)
    dev = to_device(prob)
    r = Runner(prob, dev=dev)
    rows = torch.empty((int(prob.cache_seqlens.sum()), 576), dtype=torch.int16, device="cuda")
    B.mla_debug_gather(r.plan, dev["kv_cache"], dev["block_table"], rows)
    got = rows.cpu().numpy().view(np.uint16)
    off = 0
    for b in range(prob.batch):
        L = int(prob.cache_seqlens[b])
        ref = orc.gather_sequence(prob.kv_cache, prob.block_table[b], L, page)
        assert np.array_equal(got[off:off + L], ref), f"seq {b}"
        off += L


# ----------------------------------------------------------------------------- the five workloads
def test_parity_tiny():
    prob = gen.make_config("tiny")          # fp32 out
    out, lse = run(prob)
    ref_o, ref_l = oracle(prob)
    compare(out, lse, ref_o, ref_l, what="tiny")
    compare(out, lse, ref_o, ref_l, what="tiny (fp32 bound)", tol=(F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL))


def test_parity_paged():
    prob = gen.make_config("paged")
    out, lse = run(prob)
    ref_o, ref_l = oracle(prob)
    compare(out, lse, ref_o, ref_l, what="paged")


def compare_every_sequence(out, lse, ref_out, ref_lse, what, tol=(RMSE_TOL, MAX_TOL, LSE_TOL)):
    """Every sequence of the call against the oracle: the pooled bounds over the whole output,
    and each sequence's own RMSE and max |err| held to the same bounds (the worst is printed)."""
    compare(out, lse, ref_out, ref_lse, what=what + " (all sequences)", tol=tol)
    worst = (0.0, 0.0, -1)
    for b in range(out.shape[0]):
        err = out[b] - ref_out[b]
        r, m = float(np.sqrt(np.mean(err ** 2))), float(np.max(np.abs(err)))
        assert r <= tol[0] and m <= tol[1], (what, b, r, m)
        worst = max(worst, (r, m, b))
    _say(f"  {what}: worst sequence {worst[2]}: rmse {worst[0]:.3e} max {worst[1]:.3e}")


@pytest.mark.parametrize("name", ["two_token", "long", "ragged"])
def test_parity_full_size(name):
    _say(f"generating {name}")
    prob = gen.make_config(name)
    _say(f"running {name} on the GPU")
    out, lse = run(prob)
    _say(f"oracle on all {prob.batch} sequences")
    ref_o, ref_l = oracle(prob)
    compare_every_sequence(out, lse, ref_o, ref_l, name)


# ----------------------------------------------------------------------------- edge cases
@pytest.mark.parametrize("page", [16, 48, 64, 80, 1024])
@pytest.mark.parametrize("out_fp32", [True, False])
def test_edge_lengths_nan_tails(page, out_fp32):
    lengths = [1, 15, 16, 17, 63, 64, 65, 1000]
    prob = gen.make_problem(batch=len(lengths), q_len=1, num_heads=16, page_size=page, lengths=lengths, seed=5,
                            tail="nan", extra_pages=3, out_fp32=out_fp32)
    out, lse = run(prob)
    ref_o, ref_l = oracle(prob)
    check_short_contexts(out, lse, ref_o, ref_l, out_fp32, f"edges P={page}", None if out_fp32 else softmax_abs_v(prob))


@pytest.mark.parametrize("heads,page,kv", [(128, 48, "bf16"), (128, 80, "bf16"), (32, 48, "bf16"),
                                          (64, 80, "fp8")])
def test_non_power_of_two_pages(heads, page, kv):
    """Page sizes that are multiples of 16 but not powers of two take the division in the
    page walk (powers of two take a shift): the wide kernel (128 rows), the 32-row kernel and the
    FP8 path in the wide kernel (64 rows)."""
    prob = gen.make_problem(batch=3, q_len=1, num_heads=heads, page_size=page, lengths=[page * 7 + 5, 33, 2000],
                            seed=23, tail="nan", extra_pages=2, kv_format=kv)
    out, lse = run(prob)
    ref_o, ref_l = oracle(prob)
    check_short_contexts(out, lse, ref_o, ref_l, False, f"P={page} H={heads} {kv}", softmax_abs_v(prob))


@pytest.mark.parametrize("out_fp32", [False, True])
@pytest.mark.parametrize("heads,q_len", [(16, 1), (16, 2), (32, 2), (128, 1)])
def test_single_token_returns_v_row(out_fp32, heads, q_len):
    """One cached token: its weight is exactly 1, so every row of the output is its V row, bit for
    bit (R = 16, 32, 64 and 128: each work-group width)."""
    prob = gen.make_problem(batch=4, q_len=q_len, num_heads=heads, page_size=64, lengths=[1, 1, 1, 1], seed=6,
                            tail="nan", out_fp32=out_fp32)
    out, lse = run(prob)
    for b in range(prob.batch):
        v = gen.bf16_bits_to_f32(prob.kv_cache[prob.block_table[b, 0], 0, :512]).astype(np.float64)
        assert np.array_equal(out[b], np.broadcast_to(v, out[b].shape)), f"seq {b}: out != V row"
    ref_o, ref_l = oracle(prob)
    assert np.max(np.abs(lse - ref_l)) <= LSE_TOL


def test_empty_context():
    prob = gen.make_problem(batch=3, q_len=1, num_heads=16, page_size=64, lengths=[0, 100, 0], seed=7)
    out, lse = run(prob)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    ref_o, ref_l = oracle(prob, [1])
    compare(out, lse, ref_o, ref_l, batch_idx=[1], what="L=0 neighbours")


def test_page_permutation_bit_identical():
    rng = np.random.default_rng(8)
    prob = gen.make_problem(batch=4, q_len=1, num_heads=16, page_size=64, lengths=[3000, 64, 5000, 17], seed=8,
                            extra_pages=5)
    out1, lse1 = run(prob)
    perm = rng.permutation(prob.num_pages)
    kv2 = np.empty_like(prob.kv_cache)
    kv2[perm] = prob.kv_cache
    bt2 = np.where(prob.block_table >= 0, perm[np.maximum(prob.block_table, 0)], -1).astype(np.int32)
    prob2 = gen.Problem(q=prob.q, kv_cache=kv2, block_table=bt2, cache_seqlens=prob.cache_seqlens,
                        softmax_scale=prob.softmax_scale, page_size=64)
    out2, lse2 = run(prob2)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


@pytest.mark.parametrize("force", [1, 2, 3, 4, 5, 8, 9, 16, 17, 1000])
def test_forced_split_counts_agree(force):
    """Every sequence cut into min(force, blocks) pieces: the merge reads its partials in batches
    of 4, 8 or 16 (the plan's largest piece count rounded up), so 4/5, 8/9 and 16/17 pieces sit
    on both sides of each batch size, and 1000 takes several batches of 16."""
    prob = gen.make_problem(batch=3, q_len=1, num_heads=16, page_size=64, lengths=[4096, 100, 2500], seed=9)
    out, lse = run(prob, force_splits=force)
    ref_o, ref_l = oracle(prob)
    compare(out, lse, ref_o, ref_l, what=f"force_splits={force}")


@pytest.mark.parametrize("out_fp32", [True, False])
def test_many_pieces_per_work_group(out_fp32):
    prob = gen.make_problem(batch=700, q_len=1, num_heads=16, page_size=16, lengths=None, ragged_range=(1, 80),
                            seed=10, out_fp32=out_fp32)
    r = Runner(prob, num_cus=16)            # 16 work-groups: each walks many sequences
    assert max(np.diff(r.plan.segments()[1])) > 10
    r()
    out, lse = r.results()
    ref_o, ref_l = oracle(prob)
    check_short_contexts(out, lse, ref_o, ref_l, out_fp32, "many pieces", None if out_fp32 else softmax_abs_v(prob))


@pytest.mark.parametrize("heads,rpg", [(64, 64), (32, 32), (128, 64), (128, 128)])
@pytest.mark.parametrize("out_fp32", [True, False])
def test_wide_and_32_row_kernels_many_pieces(heads, rpg, out_fp32):
    """The 32-row and wide kernels (64 and 128 rows) walking many pieces per work-group (the
    slots and exchange buffers reused from piece to piece), with empty, one-token and
    page-crossing sequences among them."""
    rng = np.random.default_rng(12)
    lengths = rng.integers(0, 300, size=90)
    lengths[::17] = 0
    lengths[5::23] = 1
    prob = gen.make_problem(batch=90, q_len=1, num_heads=heads, page_size=32, lengths=lengths.tolist(), seed=12,
                            tail="nan", out_fp32=out_fp32)
    r = Runner(prob, num_cus=24, rows_per_group=rpg)
    assert r.plan.info()["rows_per_group"] == rpg
    assert max(np.diff(r.plan.segments()[1])) > 3
    r()
    out, lse = r.results()
    ref_o, ref_l = oracle(prob)
    check_short_contexts(out, lse, ref_o, ref_l, out_fp32, f"many pieces H={heads} rpg={rpg}",
                         None if out_fp32 else softmax_abs_v(prob))


@pytest.mark.parametrize("heads,q_len", [(16, 2), (32, 1), (64, 1), (48, 1), (128, 1), (64, 2), (128, 2), (16, 9)])
def test_more_query_rows(heads, q_len):
    prob = gen.make_problem(batch=3, q_len=q_len, num_heads=heads, page_size=64, lengths=[700, 2000, 33], seed=11)
    out, lse = run(prob)
    ref_o, ref_l = oracle(prob)
    compare(out, lse, ref_o, ref_l, what=f"H={heads} S_q={q_len}")


@pytest.mark.parametrize("heads,q_len,rpg", [(16, 2, 32), (32, 1, 32), (64, 1, 64), (128, 1, 64), (16, 4, 64),
                                          (64, 2, 64), (128, 1, 16), (64, 1, 16), (128, 2, 64), (128, 2, 16),
                                          (128, 1, 128), (64, 2, 128), (128, 2, 128), (16, 8, 128)])
@pytest.mark.parametrize("out_fp32", [True, False])
def test_rows_per_group_option(heads, q_len, rpg, out_fp32):
    """Rows per work-group asked for through the plan option: the 32-row kernel, the wide kernel
    with 64 rows (two waves per 32 rows) and 128, in several row groups, and the 16-row kernel
    where a wider one would be chosen by default."""
    prob = gen.make_problem(batch=4, q_len=q_len, num_heads=heads, page_size=64, lengths=[700, 2000, 33, 1],
                            seed=18, tail="nan", extra_pages=1, out_fp32=out_fp32)
    r = Runner(prob, rows_per_group=rpg)
    assert r.plan.info()["rows_per_group"] == rpg
    r()
    out, lse = r.results()
    ref_o, ref_l = oracle(prob)
    check_short_contexts(out, lse, ref_o, ref_l, out_fp32, f"H={heads} S_q={q_len} rpg={rpg}",
                         None if out_fp32 else softmax_abs_v(prob))


def with_score_ramp(prob, slope=0.1):
    """The same problem with rope column 512 of every cached row set to slope * t (t the
    token's position in its sequence) and the queries' column 512 set to 1, so each score
    gains sigma * slope * t: the running max keeps climbing along the context."""
    kv = prob.kv_cache.copy()
    q = prob.q.copy()
    q[..., 512] = gen.f32_to_bf16_bits(np.float32(1.0))
    for b in range(prob.batch):
        t = np.arange(int(prob.cache_seqlens[b]))
        bits = gen.f32_to_bf16_bits((slope * t).astype(np.float32))
        pages, rows = prob.block_table[b, t // prob.page_size], t % prob.page_size
        if kv.dtype == np.uint8:       # fp8 rows: the rope columns are bf16 at bytes 512..639
            kv[pages, rows, 512] = (bits & 0xFF).astype(np.uint8)
            kv[pages, rows, 513] = (bits >> 8).astype(np.uint8)
        else:
            kv[pages, rows, 512] = bits
    return gen.Problem(q=q, kv_cache=kv, block_table=prob.block_table, cache_seqlens=prob.cache_seqlens,
                       softmax_scale=prob.softmax_scale, page_size=prob.page_size, out_fp32=prob.out_fp32)


@pytest.mark.parametrize("heads,q_len,rpg,kv", [(16, 1, 0, "bf16"), (16, 2, 0, "bf16"), (16, 2, 32, "bf16"),
                                             (128, 1, 0, "bf16"), (128, 1, 64, "bf16"), (16, 1, 0, "fp8"),
                                             (64, 1, 0, "fp8")])
@pytest.mark.parametrize("out_fp32", [True, False])
def test_climbing_scores_move_the_running_max(heads, q_len, rpg, kv, out_fp32):
    """Scores that grow along the context (about 31 log2 units over 3,000 tokens) with 8
    work-groups, so every wave's running max passes its lazy-rescale slack (8) several times
    in mid-stream and O and l are rescaled with weights already accumulated."""
    base = gen.make_problem(batch=3, q_len=q_len, num_heads=heads, page_size=64, lengths=[3000, 777, 1285],
                            seed=31, kv_format=kv, out_fp32=out_fp32, tail="nan", extra_pages=1)
    prob = with_score_ramp(base)
    r = Runner(prob, num_cus=8, rows_per_group=rpg)
    r()
    out, lse = r.results()
    ref_o, ref_l = oracle(prob)
    check_short_contexts(out, lse, ref_o, ref_l, out_fp32, f"climbing H={heads} S_q={q_len} rpg={rpg} {kv}",
                         None if out_fp32 else softmax_abs_v(prob))


@pytest.mark.parametrize("heads,q_len,rpg", [(128, 1, 128), (128, 2, 128), (16, 1, 16), (64, 1, 64), (32, 1, 32)])
@pytest.mark.parametrize("out_fp32", [True, False])
def test_scores_far_above_the_first_block(heads, q_len, rpg, out_fp32):
    """Scores that climb about 150 log2 units along 3,000 tokens (and fall again in one
    sequence): every piece's later scores exceed its first block's maximum by far more than
    any slack, so the 128-row kernel recomputes those pieces from their true maxima and the
    other kernels rescale many times; all must match the oracle."""
    base = gen.make_problem(batch=3, q_len=q_len, num_heads=heads, page_size=64, lengths=[3000, 1500, 1285],
                            seed=33, out_fp32=out_fp32, tail="nan", extra_pages=1)
    prob = with_score_ramp(base, slope=0.5)
    kv = prob.kv_cache.copy()                # sequence 2: the ramp reversed (the maximum comes first)
    t = np.arange(int(prob.cache_seqlens[2]))
    bits = gen.f32_to_bf16_bits((0.5 * (t[::-1])).astype(np.float32))
    kv[prob.block_table[2, t // 64], t % 64, 512] = bits
    prob = gen.Problem(q=prob.q, kv_cache=kv, block_table=prob.block_table, cache_seqlens=prob.cache_seqlens,
                       softmax_scale=prob.softmax_scale, page_size=64, out_fp32=out_fp32)
    r = Runner(prob, num_cus=8, rows_per_group=rpg)
    r()
    out, lse = r.results()
    ref_o, ref_l = oracle(prob)
    check_short_contexts(out, lse, ref_o, ref_l, out_fp32, f"steep H={heads} S_q={q_len} rpg={rpg}",
                         None if out_fp32 else softmax_abs_v(prob), lse_ulps=2)


def test_two_token_query_equals_two_single_token_calls():
    prob = gen.make_problem(batch=2, q_len=2, num_heads=16, page_size=64, lengths=[1500, 300], seed=12,
                            out_fp32=True)
    out, lse = run(prob)
    for i in range(2):
        p1 = gen.Problem(q=np.ascontiguousarray(prob.q[:, i:i + 1]), kv_cache=prob.kv_cache,
                         block_table=prob.block_table, cache_seqlens=prob.cache_seqlens,
                         softmax_scale=prob.softmax_scale, page_size=64, out_fp32=True)
        o1, l1 = run(p1)
        assert np.max(np.abs(o1[:, 0] - out[:, i])) <= 1e-5 and np.max(np.abs(l1[:, 0] - lse[:, i])) <= 1e-5


def test_out_of_range_block_table_entry_is_flagged():
    import torch
    prob = gen.make_problem(batch=2, q_len=1, num_heads=16, page_size=64, lengths=[640, 640], seed=13)
    good = Runner(prob)
    assert B.mla_read_status(good.ws) == 0
    good()
    torch.cuda.synchronize()
    assert B.mla_read_status(good.ws) == 0
    bt = prob.block_table.copy()
    bt[1, 3] = prob.num_pages + 7            # outside [0, num_pages): its 64 tokens are dropped
    bad = gen.Problem(q=prob.q, kv_cache=prob.kv_cache, block_table=bt, cache_seqlens=prob.cache_seqlens,
                      softmax_scale=prob.softmax_scale, page_size=64)
    r = Runner(bad)
    r()
    out, lse = r.results()
    assert B.mla_read_status(r.ws) & 1
    ref_o, ref_l = oracle(prob, [0])
    compare(out, lse, ref_o, ref_l, batch_idx=[0], what="unaffected sequence")
    check_dropped_page(prob, out, lse, seq=1, page_idx=3)


@pytest.mark.parametrize("heads,rpg", [(128, 0), (128, 64), (32, 32), (64, 16)])
def test_out_of_range_entry_drops_one_block(heads, rpg):
    """Page size 16 (one block per page): an out-of-range entry makes one 16-token half of a
    32-token block of the wide kernel unused (the first half in sequence 0, the second in
    sequence 1); its tokens are dropped and the status bit is set.  Unmapped pages hold NaN."""
    prob = gen.make_problem(batch=2, q_len=1, num_heads=heads, page_size=16, lengths=[640, 650], seed=22,
                            tail="nan", extra_pages=2)
    bt = prob.block_table.copy()
    bt[0, 10] = -1
    bt[1, 5] = prob.num_pages + 3
    bad = gen.Problem(q=prob.q, kv_cache=prob.kv_cache, block_table=bt, cache_seqlens=prob.cache_seqlens,
                      softmax_scale=prob.softmax_scale, page_size=16)
    r = Runner(bad, rows_per_group=rpg)
    assert r.plan.info()["rows_per_group"] == (rpg or 128)
    r()
    out, lse = r.results()
    assert B.mla_read_status(r.ws) & 1
    check_dropped_page(prob, out, lse, seq=0, page_idx=10)
    check_dropped_page(prob, out, lse, seq=1, page_idx=5)


def test_workspace_of_another_plan_is_refused():
    """Two plans, one workspace: after plan B's upload, a decode with plan A is refused on the
    host (MLA_ERR_PLAN_MISMATCH, nothing launched); plan B decodes; A decodes again after its
    own upload."""
    import torch
    pa = gen.make_problem(batch=2, q_len=1, num_heads=16, page_size=64, lengths=[3000, 500], seed=43)
    pb = gen.make_problem(batch=2, q_len=1, num_heads=16, page_size=64, lengths=[700, 5000], seed=44)
    ra, rb = Runner(pa), Runner(pb)
    ws = ra.ws if ra.ws.numel() >= rb.ws.numel() else rb.ws
    ra.ws = rb.ws = ws
    for r in (ra, rb):
        d = r.dev
        r._bound = B.BoundDecode(r.plan, d["q"], d["kv_cache"], d["block_table"], d["cache_seqlens"],
                                 r.prob.softmax_scale, r.out, r.lse, ws)
    ra.plan.upload(ws)
    rb.plan.upload(ws)
    ra.out.fill_(7.0)
    with pytest.raises(B.MlaError) as ei:
        ra()
    assert ei.value.status == B.MLA_ERR_PLAN_MISMATCH
    torch.cuda.synchronize()
    assert bool(torch.all(ra.out == 7.0))
    rb()
    out, lse = rb.results()
    compare(out, lse, *oracle(pb), what="plan B in the shared workspace")
    ra.plan.upload(ws)
    ra()
    out, lse = ra.results()
    compare(out, lse, *oracle(pa), what="plan A after its own upload")
    assert B.mla_read_status(ws) == 0


@pytest.mark.parametrize("heads", [16, 128])
def test_overwritten_plan_id_is_caught_on_the_device(heads):
    """The host record says the workspace holds the plan, but its id bytes were overwritten (as
    by another upload after a graph capture): the kernels read no schedule, out and lse stay
    as they were, and status bit 3 is set."""
    import torch
    prob = gen.make_problem(batch=2, q_len=1, num_heads=heads, page_size=64, lengths=[3000, 500], seed=45)
    r = Runner(prob)
    r.ws[8:16].zero_()
    r.out.fill_(7.0)
    r.lse.fill_(3.0)
    r()
    torch.cuda.synchronize()
    assert bool(torch.all(r.out == 7.0)) and bool(torch.all(r.lse == 3.0))
    assert B.mla_read_status(r.ws) == 8
    r.plan.upload(r.ws)                       # a fresh upload restores the id and clears the status
    r()
    out, lse = r.results()
    compare(out, lse, *oracle(prob), what="after a fresh upload")
    assert B.mla_read_status(r.ws) == 0


@pytest.mark.parametrize("heads", [16, 128])
def test_device_length_beyond_the_plan_is_flagged(heads):
    """Device cache_seqlens above the planned ones: the extra tokens are not attended (the
    result is the plan's), and status bit 2 is set; shorter device lengths are honoured
    without a flag."""
    import torch
    prob = gen.make_problem(batch=3, q_len=1, num_heads=heads, page_size=64, lengths=[3000, 500, 64], seed=46,
                            extra_pages=4)
    r = Runner(prob)
    longer = prob.cache_seqlens.copy()
    longer[1] += 100                          # past the sequence's mapped pages: never read
    r.dev["cache_seqlens"].copy_(torch.from_numpy(longer.astype(np.int32)))
    r()
    out, lse = r.results()
    assert B.mla_read_status(r.ws) == 4
    compare(out, lse, *oracle(prob), what="clipped to the planned lengths")
    r.plan.upload(r.ws)
    shorter = prob.cache_seqlens.copy()
    shorter[0] -= 1000
    r.dev["cache_seqlens"].copy_(torch.from_numpy(shorter.astype(np.int32)))
    r()
    out, lse = r.results()
    assert B.mla_read_status(r.ws) == 0
    ref_o, ref_l = orc.decode(prob.q, prob.kv_cache, prob.block_table, shorter, prob.softmax_scale, prob.page_size)
    compare(out, lse, ref_o, ref_l, what="shorter device lengths")


def check_dropped_page(prob, out, lse, seq, page_idx, tol=(RMSE_TOL, MAX_TOL, LSE_TOL)):
    """Sequence `seq` must equal attention over its tokens outside table entry `page_idx`."""
    P, L = prob.page_size, int(prob.cache_seqlens[seq])
    keep = [t for t in range(L) if t // P != page_idx]
    rows = orc.widen_rows(orc.gather_sequence(prob.kv_cache, prob.block_table[seq], L, P)[keep])
    R = prob.q_len * prob.num_heads
    q = orc.widen_bf16(prob.q[seq]).reshape(R, -1)
    ref_o, ref_l = orc.attend(q, rows, rows[:, :512], prob.softmax_scale)
    ro = ref_o.reshape(out[seq].shape)
    rl = ref_l.reshape(lse[seq].shape)
    err = out[seq] - ro
    rmse, mx, le = float(np.sqrt(np.mean(err ** 2))), float(np.max(np.abs(err))), float(np.max(np.abs(lse[seq] - rl)))
    _say(f"  dropped page {page_idx} of sequence {seq}: rmse {rmse:.2e} max {mx:.2e} lse {le:.2e}")
    assert rmse <= tol[0] and mx <= tol[1] and le <= tol[2]


def test_repeated_calls_are_deterministic():
    prob = gen.make_problem(batch=4, q_len=1, num_heads=16, page_size=64, lengths=[9000, 100, 5000, 64], seed=14)
    r = Runner(prob)
    r()
    o1, l1 = r.results()
    for _ in range(3):
        r()
        o2, l2 = r.results()
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_two_streams_at_once():
    """Two decodes with their own plans and workspaces, launched on two streams without a
    synchronisation between them (the library keeps no per-call state outside the
    workspace), each matching the oracle."""
    import torch
    p1 = gen.make_problem(batch=3, q_len=1, num_heads=16, page_size=64, lengths=[5000, 70, 2600], seed=41)
    p2 = gen.make_problem(batch=2, q_len=2, num_heads=64, page_size=16, lengths=[3333, 900], seed=42,
                          kv_format="fp8")
    r1, r2 = Runner(p1), Runner(p2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        r1(stream=s1)
        r2(stream=s2)
    torch.cuda.synchronize()
    for prob, r, what in ((p1, r1, "stream 1"), (p2, r2, "stream 2 (fp8)")):
        out, lse = r.results()
        ref_o, ref_l = oracle(prob)
        compare(out, lse, ref_o, ref_l, what=what)


def test_graph_capture_replays_match_eager():
    """The decode launches are capturable in a HIP graph (no memset nodes); every replay,
    with other GPU work in between, gives the eager result bit for bit."""
    import torch
    prob = gen.make_problem(batch=4, q_len=1, num_heads=16, page_size=64, lengths=[9000, 100, 5000, 64], seed=15)
    r = Runner(prob)
    r()
    ref_o, ref_l = r.results()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            r(stream=side)
    torch.cuda.current_stream().wait_stream(side)
    junk = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        r.out.zero_()
        r.lse.zero_()
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o, l = r.results()
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l), f"replay {i}"


def _spread_beyond_4gib(prob, big_pages, seed):
    """The same problem with its pages placed at physical pages of a cache of big_pages
    pages (> 4 GiB): most referenced pages land past the 4-GiB byte offset, a few near the
    start.  Returns (problem whose num_pages is big_pages, device tensors)."""
    import dataclasses
    import torch
    rng = np.random.default_rng(seed)
    n = prob.num_pages
    page_bytes = prob.kv_cache[0].nbytes
    first_high = (4 << 30) // page_bytes + 1
    assert big_pages - first_high >= n
    remap = rng.choice(np.arange(first_high, big_pages), size=n, replace=False)
    remap[: min(2, n)] = np.arange(min(2, n))                 # a couple at the start of the cache
    bt = prob.block_table
    bt_big = np.where(bt >= 0, remap[np.clip(bt, 0, n - 1)], -1).astype(np.int32)
    # a cache array that reports big_pages pages without holding them (only its shape is used)
    fake = np.lib.stride_tricks.as_strided(prob.kv_cache[:1], shape=(big_pages,) + prob.kv_cache.shape[1:],
                                           strides=(0,) + prob.kv_cache.strides[1:], writeable=False)
    big_prob = dataclasses.replace(prob, kv_cache=fake, block_table=bt_big)
    small = to_device(prob)
    big = torch.empty((big_pages,) + tuple(small["kv_cache"].shape[1:]), dtype=small["kv_cache"].dtype,
                      device="cuda")
    assert big.numel() * big.element_size() > (4 << 30)
    big.index_copy_(0, torch.from_numpy(remap).to("cuda"), small["kv_cache"])
    dev = dict(small, kv_cache=big, block_table=torch.from_numpy(bt_big).to("cuda"))
    return big_prob, dev


@pytest.mark.parametrize("heads,rpg,kv", [(16, 16, "bf16"), (64, 64, "bf16"), (128, 128, "bf16"), (16, 16, "fp8")])
def test_cache_beyond_4gib(heads, rpg, kv):
    """A cache larger than 4 GiB with the sequences' pages past the 4-GiB byte offset: the
    page walk and the DMA addresses are 64-bit.  The result equals the same problem on a
    compact cache bit for bit, and the oracle within the fp32-path bounds."""
    import torch
    prob = gen.make_problem(batch=3, q_len=1, num_heads=heads, page_size=64, lengths=[3000, 700, 65],
                            seed=19, out_fp32=True, kv_format=kv)
    big_pages = 65536 if kv == "bf16" else 110000
    _say(f"  cache beyond 4 GiB: heads={heads} rpg={rpg} kv={kv} pages={big_pages}")
    big_prob, dev = _spread_beyond_4gib(prob, big_pages, seed=19)
    r_big = Runner(big_prob, dev=dev, rows_per_group=rpg)
    r_big()
    out_b, lse_b = r_big.results()
    r_small = Runner(prob, rows_per_group=rpg)
    r_small()
    out_s, lse_s = r_small.results()
    assert np.array_equal(out_b, out_s) and np.array_equal(lse_b, lse_s)
    ref_o, ref_l = oracle(prob)
    compare(out_b, lse_b, ref_o, ref_l, what=f"beyond 4 GiB {kv}", tol=(F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL))
    del r_big, dev
    torch.cuda.empty_cache()


_MILLION = {}


@pytest.mark.parametrize("devplan", [False, True])
def test_one_sequence_of_a_million_tokens(devplan):
    """One sequence of 2^20 tokens: the planner (or the device schedule) cuts it over every
    work-group and the merge combines a few hundred partial results."""
    from mla_decode_attention_paged_amd.device import DevplanRunner
    if not _MILLION:                      # inputs and oracle shared by both cases
        p = gen.make_problem(batch=1, q_len=1, num_heads=16, page_size=64, lengths=[1 << 20], seed=23, out_fp32=True)
        _MILLION.update(prob=p, ref=oracle(p))
    prob = _MILLION["prob"]
    ref_o, ref_l = _MILLION["ref"]
    _say(f"  one sequence of {1 << 20} tokens, devplan={devplan}")
    if devplan:
        r = DevplanRunner(prob)
    else:
        r = Runner(prob)
        assert r.plan.info()["num_partials"] >= 200
    r()
    out, lse = r.results()
    compare(out, lse, ref_o, ref_l, what="2^20 tokens", tol=(F32_RMSE_TOL, F32_MAX_TOL, F32_LSE_TOL))
    if devplan:
        _MILLION.clear()
