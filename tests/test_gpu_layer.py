"""The steps around the decode on the HIP path (through the C-ABI) against the fp64 oracle.

Bars:
  rope columns     -- bit-exact bf16 (both sides evaluate the rotation in float64 and round
                      once); a 1-ulp difference is accepted only where the float64 value lies
                      within 1e-9 (relative) of a bf16 rounding midpoint.
  fp8 cache bytes  -- bit-exact (codes and scales are integer decisions taken on exact values).
  bf16 latent copy -- bit-exact.
  MFMA products    -- |got - ref| <= (bf16 output: half an ulp of ref) + 2^-14 * sum_i |a_i b_i|:
                      float32 accumulation of K <= 512 exact bf16 products (K * 2^-24) plus, for
                      a float32 input split as hi + lo, its 2^-17 relative residual.
  whole layer step -- append -> query preparation -> causal decode -> output projection
                      against the decompressed-attention oracle: RMSE <= 1e-3, max <= 1e-2.
"""
import numpy as np
import pytest

from mla_decode_attention_paged_amd import binding as B
from mla_decode_attention_paged_amd import inputs as gen
from mla_decode_attention_paged_amd.device import Runner, layer_to_device, problem_struct, to_device
from oracle import mla_layer as L
from oracle import mla_oracle as orc
from tests.test_gpu_parity import MAX_TOL, RMSE_TOL, _say, bf16_half_ulp

pytestmark = pytest.mark.gpu

ROPE_BASE = 10000.0


def _bits(t):
    import torch
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _positions(batch, q_len, rng, max_pos):
    pos = rng.integers(0, max_pos, size=(batch, q_len)).astype(np.int32)
    pos.flat[0] = 0
    if pos.size > 1:
        pos.flat[-1] = max_pos - 1
    return pos


def check_bf16_near_exact(got_bits, ref, what):
    """got bf16 bits equal the round-to-nearest-even of the float64 ref, except at near-ties."""
    want = L._f64_to_bf16_bits(ref)
    diff = got_bits != want
    if np.any(diff):
        g = orc.widen_bf16(got_bits[diff])
        w = orc.widen_bf16(want[diff])
        r = ref[diff]
        mid = (g + w) / 2
        near_tie = np.abs(r - mid) <= 1e-9 * np.abs(r)
        one_ulp = np.abs(g - w) <= 2 * bf16_half_ulp(r) * 1.0001
        assert np.all(near_tie & one_ulp), f"{what}: {int(diff.sum())} values differ, e.g. {g[:4]} vs {w[:4]}"
    _say(f"  {what}: {got_bits.size} values, {int(diff.sum())} near-tie differences")


def check_mfma(got, ref, abs_sum, bf16_out, what):
    bound = 2.0 ** -14 * abs_sum + (bf16_half_ulp(ref) if bf16_out else 0.0)
    excess = np.abs(got - ref) - bound
    _say(f"  {what}: max |err| {np.max(np.abs(got - ref)):.3e}, worst margin {np.max(excess):.3e}")
    assert np.all(excess <= 0), what


SHAPES = [(1, 1, 16), (3, 2, 16), (16, 1, 16), (5, 7, 16), (4, 1, 128), (2, 2, 64), (32, 2, 16), (2, 2, 128)]


@pytest.mark.parametrize("batch,q_len,heads", SHAPES)
def test_q_absorb(batch, q_len, heads):
    import torch
    rng = np.random.default_rng(batch * 1000 + q_len * 10 + heads)
    li = gen.make_layer_inputs(batch, q_len, heads, seed=int(rng.integers(1 << 30)))
    pos = _positions(batch, q_len, rng, 65536)
    d = layer_to_device(li)
    prob = B.make_problem(batch, q_len, heads, 64, 1, 1)
    q_out = torch.empty((batch, q_len, heads, 576), dtype=torch.bfloat16, device="cuda")
    B.mla_q_absorb(prob, d["q_nope"], d["q_pe"], d["w_uk"], torch.from_numpy(pos).cuda(), ROPE_BASE, q_out)
    got = _bits(q_out)
    ref = L.q_absorb(li.q_nope, li.q_pe, li.w_uk, pos, ROPE_BASE)
    abs_sum = np.einsum("bshd,hed->bshe", np.abs(orc.widen_bf16(li.q_nope)), np.abs(orc.widen_bf16(li.w_uk)))
    check_mfma(orc.widen_bf16(got[..., :512]), ref[..., :512], abs_sum, True, f"q latent B={batch} S={q_len} H={heads}")
    check_bf16_near_exact(got[..., 512:], ref[..., 512:], f"q rope B={batch} S={q_len} H={heads}")


@pytest.mark.parametrize("batch,q_len,heads", SHAPES)
@pytest.mark.parametrize("fp32", [False, True])
def test_out_absorb(batch, q_len, heads, fp32):
    import torch
    if (q_len * heads) % 16 or q_len * heads > 256:
        pytest.skip("q_len * heads outside the decode's row range")
    rng = np.random.default_rng(batch * 999 + q_len * 7 + heads + fp32)
    li = gen.make_layer_inputs(batch, q_len, heads, seed=int(rng.integers(1 << 30)))
    d = layer_to_device(li)
    lat = rng.standard_normal((batch, q_len, heads, 512)).astype(np.float32)
    if fp32:
        lat_t = torch.from_numpy(lat).cuda()
        lat_ref = lat.astype(np.float64)
    else:
        bits = gen.f32_to_bf16_bits(lat)
        lat_t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        lat_ref = orc.widen_bf16(bits)
    prob = B.make_problem(batch, q_len, heads, 64, 1, 1, out_fp32=fp32)
    o = torch.empty((batch, q_len, heads, 128), dtype=torch.float32 if fp32 else torch.bfloat16, device="cuda")
    B.mla_out_absorb(prob, lat_t, d["w_uv"], o)
    torch.cuda.synchronize()
    got = o.cpu().numpy().astype(np.float64) if fp32 else orc.widen_bf16(_bits(o))
    ref = L.out_absorb(lat_ref, li.w_uv)
    abs_sum = np.einsum("bshe,hve->bshv", np.abs(lat_ref), np.abs(orc.widen_bf16(li.w_uv)))
    check_mfma(got, ref, abs_sum, not fp32, f"out B={batch} S={q_len} H={heads} fp32={fp32}")


def _append_case(kv_format, page_size, lengths, q_len, seed):
    prob = gen.make_problem(batch=len(lengths), q_len=q_len, num_heads=16, page_size=page_size, lengths=lengths,
                            seed=seed, kv_format=kv_format, extra_pages=1)
    li = gen.make_layer_inputs(prob.batch, q_len, 16, seed=seed + 1)
    pos = (prob.cache_seqlens[:, None] - q_len + np.arange(q_len)[None, :]).astype(np.int32)
    return prob, li, pos


@pytest.mark.parametrize("kv_format", ["bf16", "fp8"])
@pytest.mark.parametrize("page_size,q_len", [(16, 1), (16, 2), (64, 2), (64, 4)])
def test_kv_append(kv_format, page_size, q_len):
    import torch
    prob, li, pos = _append_case(kv_format, page_size, [q_len, 17, 64, 65, 1000], q_len, seed=40 + page_size + q_len)
    dev = to_device(prob)
    d = layer_to_device(li)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = problem_struct(prob)
    B.mla_kv_append(p, d["c_kv"], d["k_pe"], torch.from_numpy(pos).cuda(), dev["block_table"], ROPE_BASE,
                    dev["kv_cache"], status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = dev["kv_cache"].cpu().view(torch.uint8).numpy().reshape(prob.num_pages, page_size, -1)
    want_kv = L.append_rows(prob.kv_cache, prob.block_table, li.c_kv, li.k_pe, pos, kv_format, ROPE_BASE)
    want = np.ascontiguousarray(want_kv).view(np.uint8).reshape(got.shape)
    rope = slice(512, 640) if kv_format == "fp8" else slice(1024, 1152)
    other = np.ones(got.shape[-1], dtype=bool)
    other[rope] = False
    assert np.array_equal(got[..., other], want[..., other]), "latent bytes / scales / untouched rows differ"
    # rope columns: bit-exact up to near-ties of the float64 rotation
    ref = np.stack([L.rope(orc.widen_bf16(li.k_pe[b, i]), pos[b, i], ROPE_BASE)
                    for b in range(prob.batch) for i in range(q_len)])
    got_rows = np.stack([got[prob.block_table[b, pos[b, i] // page_size], pos[b, i] % page_size]
                         for b in range(prob.batch) for i in range(q_len)])
    check_bf16_near_exact(np.ascontiguousarray(got_rows[:, rope]).view(np.uint16), ref, f"k rope {kv_format}")


def test_kv_append_out_of_range_positions():
    """Positions outside the table, or pages outside the cache, write nothing and raise bit 1."""
    import torch
    prob, li, pos = _append_case("bf16", 16, [5, 40, 33, 20], 2, seed=77)
    bt = prob.block_table.copy()
    pos[0, 0] = prob.max_pages_per_seq * 16        # one past the table
    pos[0, 1] = -1
    pos[1, 0] = 5
    pos[1, 1] = 16 * 2 + 2                         # its table entry 2 now points outside the cache
    bt[1, 2] = prob.num_pages
    bt[2, pos[2, 0] // 16] = -5                    # entry of token (2, 0) only
    prob.block_table = bt
    keep = np.array([[(0 <= pos[b, i] < prob.max_pages_per_seq * 16)
                      and 0 <= bt[b, pos[b, i] // 16] < prob.num_pages for i in range(2)] for b in range(prob.batch)])
    assert keep.sum() == 4, keep
    dev = to_device(prob)
    d = layer_to_device(li)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.mla_kv_append(problem_struct(prob), d["c_kv"], d["k_pe"], torch.from_numpy(pos).cuda(), dev["block_table"],
                    ROPE_BASE, dev["kv_cache"], status)
    torch.cuda.synchronize()
    assert int(status.item()) == 2
    got = dev["kv_cache"].cpu().view(torch.int16).numpy().view(np.uint16)
    changed = np.any(got.reshape(-1, 576) != prob.kv_cache.reshape(-1, 576), axis=1)
    assert changed.sum() == int(keep.sum()), (changed.sum(), keep.sum())
    for b in range(prob.batch):
        for i in range(2):
            if keep[b, i]:
                r = got[bt[b, pos[b, i] // 16], pos[b, i] % 16]
                assert np.array_equal(r[:512], li.c_kv[b, i])


@pytest.mark.parametrize("kv_format", ["bf16", "fp8"])
@pytest.mark.parametrize("heads,q_len", [(16, 1), (16, 2), (64, 2), (128, 1)])
def test_layer_step_matches_decompressed_attention(kv_format, heads, q_len):
    """Append the new tokens, prepare the query, decode causally, project the output."""
    import torch
    lengths = [q_len, 40, 300, 1100]
    prob = gen.make_problem(batch=len(lengths), q_len=q_len, num_heads=heads, page_size=64, lengths=lengths,
                            seed=90 + heads + q_len, kv_format=kv_format, out_fp32=True)
    li = gen.make_layer_inputs(prob.batch, q_len, heads, seed=91 + heads + q_len)
    pos = (prob.cache_seqlens[:, None] - q_len + np.arange(q_len)[None, :]).astype(np.int32)
    dev = to_device(prob)
    d = layer_to_device(li)
    p = problem_struct(prob, causal=True)
    pos_t = torch.from_numpy(pos).cuda()
    B.mla_kv_append(p, d["c_kv"], d["k_pe"], pos_t, dev["block_table"], ROPE_BASE, dev["kv_cache"])
    B.mla_q_absorb(p, d["q_nope"], d["q_pe"], d["w_uk"], pos_t, ROPE_BASE, dev["q"])
    r = Runner(prob, dev=dev, causal=True)
    out, _ = r()
    o = torch.empty((prob.batch, q_len, heads, 128), dtype=torch.float32, device="cuda")
    B.mla_out_absorb(p, out, d["w_uv"], o)
    torch.cuda.synchronize()
    got = o.cpu().numpy().astype(np.float64)

    kv = L.append_rows(prob.kv_cache, prob.block_table, li.c_kv, li.k_pe, pos, kv_format, ROPE_BASE)
    ref = np.zeros_like(got)
    for b in range(prob.batch):
        rows = orc.widen_rows(orc.gather_sequence(kv, prob.block_table[b], int(prob.cache_seqlens[b]), 64))
        for i in range(q_len):
            vis = int(pos[b, i]) + 1          # causal: token i sees positions <= its own
            ref[b, i] = L.decompressed_attention(li.q_nope[b, i:i + 1], li.q_pe[b, i:i + 1], rows[:vis, :512],
                                                 rows[:vis, 512:], li.w_uk, li.w_uv, prob.softmax_scale,
                                                 pos[b, i:i + 1], ROPE_BASE)[0]
    err = got - ref
    rmse, mx = float(np.sqrt(np.mean(err ** 2))), float(np.max(np.abs(err)))
    _say(f"  layer {kv_format} H={heads} S_q={q_len}: rmse {rmse:.2e} max {mx:.2e} (|ref| max {np.abs(ref).max():.2f})")
    assert rmse <= RMSE_TOL and mx <= MAX_TOL
