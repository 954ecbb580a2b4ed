"""The fp64 oracle against its pins (CPU only)."""
import json
import os
from decimal import Decimal, localcontext

import numpy as np
import pytest

from mla_decode_attention_paged_amd import inputs as gen
from oracle import mla_oracle as orc
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_widen_bf16_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    w = orc.widen_bf16(bits[finite])
    for b, v in zip(bits[finite][::997], w[::997]):
        assert pins._bf16_to_decimal(int(b)) == Decimal(float(v))


def test_gather_bit_exact_roundtrip():
    """Pin P-1: scatter contiguous rows into permuted pages, gather them back."""
    rng = np.random.default_rng(1)
    for P in (16, 64, 1024):
        lengths = [1, P - 1, P, P + 1, 3 * P + 7]
        rows = [rng.integers(0, 1 << 16, size=(L, 576)).astype(np.uint16) for L in lengths]
        npages = sum((L + P - 1) // P for L in lengths) + 2
        perm = rng.permutation(npages)
        kv = np.full((npages, P, 576), 0xFFFF, dtype=np.uint16)
        bt = np.full((len(lengths), max((L + P - 1) // P for L in lengths)), -1, dtype=np.int32)
        off = 0
        for b, L in enumerate(lengths):
            for j in range((L + P - 1) // P):
                bt[b, j] = perm[off]
                seg = rows[b][j * P:(j + 1) * P]
                kv[perm[off], :seg.shape[0]] = seg
                off += 1
        for b, L in enumerate(lengths):
            got = orc.gather_sequence(kv, bt[b], L, P)
            assert got.dtype == np.uint16 and np.array_equal(got, rows[b])


def test_pin_decimal_brute_force():
    worst = pins.decimal_brute_force(orc.decode)
    assert worst <= pins.TOL


def test_pin_single_token():
    pins.single_token(orc.decode)


def test_pin_equal_scores():
    pins.equal_scores(orc.decode)


def test_pin_shift_invariance():
    pins.shift_invariance(orc.decode)


def test_pin_page_permutation():
    pins.page_permutation(orc.decode)


def test_pin_decomposition():
    pins.decomposition(orc.decode)


def test_pin_sdpa_special_case():
    pins.sdpa_special_case(orc.decode)


def test_pin_split_combine():
    pins.split_combine(orc.attend, orc.combine)
    # and the convenience wrapper
    rng = np.random.default_rng(5)
    k = rng.standard_normal((90, 576))
    q = rng.standard_normal((4, 576))
    o1, l1 = orc.attend(q, k, k[:, :512], 0.07)
    o2, l2 = orc.split_attend(q, k, k[:, :512], 0.07, [7, 40, 41])
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_empty_context():
    q = np.zeros((2, 1, 16, 576), np.uint16)
    kv = np.zeros((1, 16, 576), np.uint16)
    bt = np.array([[0], [-1]], np.int32)
    out, lse = orc.decode(q, kv, bt, np.array([1, 0], np.int32), 0.1, 16)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(out[0]))


def test_nan_tails_never_read():
    p = gen.make_problem(batch=3, q_len=1, num_heads=16, page_size=16, lengths=[5, 16, 21], seed=9,
                         tail="nan", extra_pages=2)
    out, lse = orc.decode(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, 16)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    # and the poisoned rows really are NaN
    assert np.isnan(gen.bf16_bits_to_f32(p.kv_cache[p.block_table[0, 0], 5])).all()


def _dec_attend(Q, K, V, scale):
    with localcontext() as ctx:
        ctx.prec = 40
        out, lse = [], []
        for q in Q:
            s = [Decimal(str(scale)) * sum(Decimal(str(a)) * Decimal(str(b)) for a, b in zip(q, k)) for k in K]
            m = max(s)
            ls = m + sum((x - m).exp() for x in s).ln()
            w = [(x - ls).exp() for x in s]
            out.append([float(sum(w[t] * Decimal(str(V[t][d])) for t in range(len(K)))) for d in range(len(V[0]))])
            lse.append(float(ls))
    return np.array(out), np.array(lse)


def test_golden_js_toy_inputs():
    """The page's own 3-token example: the oracle's softmax core on the page's inputs.

    The printed output table on that page is not softmax attention (its rows
    do not sum to 1 although every V row does); only the inputs are used.
    """
    g = json.load(open(os.path.join(GOLDEN, "js_toy.json")))
    Q, K, V = (np.array(g[k], dtype=np.float64) for k in ("Q", "K", "V"))
    out, lse = orc.attend(Q, K, V, g["scale"])
    ref_out, ref_lse = _dec_attend(g["Q"], g["K"], g["V"], g["scale"])
    assert np.max(np.abs(out - ref_out)) < 1e-12 and np.max(np.abs(lse - ref_lse)) < 1e-12
    # convex combination of rows that each sum to 1
    assert np.allclose(out.sum(axis=1), 1.0, atol=1e-14)
    printed = np.array(g["printed_output"])
    assert np.all(np.abs(printed.sum(axis=1) - 1.0) > 0.03), "printed table unexpectedly consistent"
    # row 0 by hand: scores 0.32, 0.24, 0.55
    s = np.array([0.32, 0.24, 0.55])
    w = np.exp(s) / np.exp(s).sum()
    assert np.allclose(out[0], w @ V, atol=1e-14)


def test_configs_shapes_small():
    p = gen.make_config("tiny")
    assert p.q.shape == (1, 1, 16, 576) and p.kv_cache.shape == (1, 1024, 576)
    assert p.block_table.tolist() == [[0]] and p.out_fp32
    out, lse = orc.decode(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, p.page_size)
    assert out.shape == (1, 1, 16, 512) and np.all(np.isfinite(out))


def test_ragged_lengths_drawn_in_range():
    p = gen.make_problem(batch=64, q_len=1, num_heads=16, page_size=64, lengths=None,
                         ragged_range=(16, 1024), seed=4)
    assert p.cache_seqlens.min() >= 16 and p.cache_seqlens.max() <= 1024
    used = np.sort(p.block_table[p.block_table >= 0])
    assert np.array_equal(used, np.arange(p.num_pages))


def test_pin_causal_decimal():
    pins.causal_decimal(orc.decode)


def test_pin_causal_decomposition():
    pins.causal_decomposition(orc.decode)


def test_pin_fp8_decoder_spec_values():
    pins.fp8_decoder_spec_values(orc.decode_e4m3)


def test_pin_fp8_decoder_matches_torch():
    pins.fp8_decoder_matches_torch(orc.decode_e4m3)


def test_pin_fp8_scale_exponent_only():
    pins.fp8_scale_exponent_only(orc.widen_fp8_rows)


def test_pin_fp8_decimal_brute_force():
    pins.fp8_decimal_brute_force(orc.decode)


def test_pin_fp8_matches_bf16_cache():
    pins.fp8_matches_bf16_cache(orc.decode)


def test_fp8_generator_rows_are_valid():
    """The generated fp8 rows: finite codes, power-of-two scales, N(0,1)-like latent values."""
    p = gen.make_problem(batch=2, q_len=1, num_heads=16, page_size=64, lengths=[100, 64], seed=44,
                         kv_format="fp8")
    rows = p.kv_cache.reshape(-1, 656)
    assert not np.any((rows[:, :512] & 0x7F) == 0x7F)
    sc = np.ascontiguousarray(rows[:, 640:656]).view(np.float32)
    assert np.all(sc == np.exp2(np.round(np.log2(sc))))
    w = orc.widen_fp8_rows(rows)
    assert 0.8 < np.std(w[:, :512]) < 1.2 and 0.8 < np.std(w[:, 512:]) < 1.2
