"""Pins for the oracle of the steps around the decode (oracle/mla_layer.py).

  rope_*          -- position 0 is the identity; each pair keeps its length; scores
                     depend only on the position difference; pair i at position p is
                     the plane rotation by p * base^(-2i/64) (written out with math).
  absorption      -- absorbed query over latent rows, then the value up-projection,
                     equals attention over explicitly decompressed per-head keys and
                     values (the low-rank compression of the FlashMLA-on-Ascend post).
  fp8 encoding    -- the E4M3 encoder against torch's float8_e4m3fn, every finite code
                     round-trips, ties go to the even code; the group exponent is the
                     smallest e >= -126 with max|x| <= 448 * 2^e.
  append          -- the latent part of a bf16 row is the input bits; an fp8 row decodes
                     to the input within half an E4M3 step; the row lands in its page.
"""
from __future__ import annotations

import math

import numpy as np

from mla_decode_attention_paged_amd import inputs as gen
from oracle import mla_layer as L
from oracle import mla_oracle as orc


def rope_pins(rope):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    assert np.allclose(rope(x, 0), x, atol=0, rtol=0)
    y = rope(x, 123.0)
    n0 = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    n1 = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    assert np.max(np.abs(n0 - n1)) < 1e-12
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n, d in ((5, 2, 7), (1000, 3, 50), (0, 9, 11)):
        a = float(rope(q, m) @ rope(k, n))
        b = float(rope(q, m + d) @ rope(k, n + d))
        assert abs(a - b) < 1e-9, (m, n, d, a, b)
    for i, p in ((0, 1), (5, 17), (31, 4095)):
        ang = p * 10000.0 ** (-2.0 * i / 64.0)
        v = np.zeros(64)
        v[2 * i], v[2 * i + 1] = 0.6, -0.8
        w = rope(v, p)
        assert abs(w[2 * i] - (0.6 * math.cos(ang) + 0.8 * math.sin(ang))) < 1e-12
        assert abs(w[2 * i + 1] - (0.6 * math.sin(ang) - 0.8 * math.cos(ang))) < 1e-12
        assert np.count_nonzero(w) <= 2


def absorption_pin(q_absorb, out_absorb, decode):
    B, S, H, P = 2, 2, 4, 16
    li = gen.make_layer_inputs(B, S, H, seed=3)
    prob = gen.make_problem(batch=B, q_len=S, num_heads=H, page_size=P, lengths=[37, 5], seed=4)
    positions = np.stack([prob.cache_seqlens - S + i for i in range(S)], axis=1)
    q = q_absorb(li.q_nope, li.q_pe, li.w_uk, positions)                 # float64 [B, S, H, 576]
    for b in range(B):
        Lb = int(prob.cache_seqlens[b])
        rows = orc.widen_bf16(orc.gather_sequence(prob.kv_cache, prob.block_table[b], Lb, P))
        s = prob.softmax_scale * np.einsum("shd,td->sht", q[b], rows)
        p = np.exp(s - s.max(axis=-1, keepdims=True))
        p /= p.sum(axis=-1, keepdims=True)
        out_latent = np.einsum("sht,td->shd", p, rows[:, :512])
        o = out_absorb(out_latent[None], li.w_uv)[0]
        ref = L.decompressed_attention(li.q_nope[b], li.q_pe[b], rows[:, :512], rows[:, 512:], li.w_uk, li.w_uv,
                                       prob.softmax_scale, positions[b])
        assert np.max(np.abs(o - ref)) < 1e-10, np.max(np.abs(o - ref))


def fp8_encoding_pins(encode, group_exponent):
    import torch
    rng = np.random.default_rng(5)
    x = np.clip(rng.standard_normal(20000) * 60, -448, 448)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode(x), t)
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.decode_e4m3(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(encode(vals[fin]), codes[fin])
    # ties: the midpoint of 1.0 (0x38, even) and 1.125 (0x39) rounds to 1.0; of 1.125 and 1.25 to 1.25
    assert encode(np.array([1.0625]))[0] == 0x38 and encode(np.array([1.1875]))[0] == 0x3A
    for amax, e in ((448.0, 0), (448.0001, 1), (224.0, -1), (224.5, 0), (1.0, -8), (1.75, -8), (1.76, -7), (0.0, 0),
                    (2.0 ** -130, -126), (448.0 * 2.0 ** -126, -126), (2.0 ** -117, -125)):
        assert group_exponent(amax) == e, (amax, group_exponent(amax), e)


def append_pins(append_rows):
    B, S, H, P = 2, 2, 4, 16
    li = gen.make_layer_inputs(B, S, H, seed=6)
    for fmt in ("bf16", "fp8"):
        prob = gen.make_problem(batch=B, q_len=S, num_heads=H, page_size=P, lengths=[20, 33], seed=7, kv_format=fmt)
        positions = np.stack([prob.cache_seqlens - S + i for i in range(S)], axis=1)
        kv = append_rows(prob.kv_cache, prob.block_table, li.c_kv, li.k_pe, positions, fmt)
        changed = np.any(kv.reshape(kv.shape[0] * P, -1) != prob.kv_cache.reshape(kv.shape[0] * P, -1), axis=1)
        assert changed.sum() <= B * S
        for b in range(B):
            for i in range(S):
                pos = int(positions[b, i])
                row = kv[prob.block_table[b, pos // P], pos % P]
                want_pe = L.rope(orc.widen_bf16(li.k_pe[b, i]), pos)
                if fmt == "bf16":
                    assert np.array_equal(row[:512], li.c_kv[b, i])
                    got_pe = orc.widen_bf16(row[512:])
                else:
                    wide = orc.widen_fp8_rows(row[None])[0]
                    x = orc.widen_bf16(li.c_kv[b, i])
                    sc = np.ascontiguousarray(row[640:656]).view(np.float32)
                    assert np.all(sc == np.exp2(np.round(np.log2(sc))))
                    for g in range(4):
                        grp = np.abs(x[128 * g:128 * (g + 1)]) / sc[g]
                        assert grp.max() <= 448 and (grp.max() > 224 or grp.max() == 0)
                    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))) / 8
                    assert np.all(np.abs(wide[:512] - x) <= np.maximum(step / 2, 2.0 ** -10 * np.repeat(sc, 128)) + 1e-12)
                    got_pe = wide[512:]
                assert np.max(np.abs(got_pe - want_pe) / np.maximum(np.abs(want_pe), 1e-3)) <= 2.0 ** -8


def bf16_rounding_pins(to_bf16_bits):
    """float64 -> bf16 rounding to nearest, ties to even, in one step.  The reference here is
    the definition itself, written independently: the two bf16 neighbours of x from the sorted
    table of every finite positive bf16 value, their distances to x (exact in float64 by
    Sterbenz's lemma, as the neighbours lie within a factor two of x), the nearer one, and on
    a tie the one with the even code.  Exact midpoints must go to the even code; values a
    sixteenth of a float32 unit off a midpoint must go to the nearer side (rounding through
    float32 first would land them on the midpoint)."""
    codes = np.arange(0x0080, 0x7F80, dtype=np.uint16)           # positive normal bf16 values
    vals = orc.widen_bf16(codes)

    def reference(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        i = np.searchsorted(vals, a, side="right") - 1            # vals[i] <= a < vals[i + 1]
        lo, hi = vals[i], vals[i + 1]
        dl, dh = a - lo, hi - a
        even_lo = (codes[i] & 1) == 0
        pick = np.where(dl < dh, codes[i], np.where(dh < dl, codes[i + 1], np.where(even_lo, codes[i], codes[i + 1])))
        return (pick | np.where(x < 0, 0x8000, 0)).astype(np.uint16)

    rng = np.random.default_rng(11)
    k = np.concatenate([np.arange(0x3E00, 0x4200, dtype=np.uint16), rng.integers(0x0100, 0x7F00, 4000).astype(np.uint16)])
    lo, hi = orc.widen_bf16(k), orc.widen_bf16(k + 1)
    mid = (lo + hi) / 2.0                                       # exact in float64
    ulp = hi - lo
    want_mid = np.where(k % 2 == 0, k, k + 1).astype(np.uint16)
    assert np.array_equal(to_bf16_bits(mid), want_mid), "exact midpoints must round to the even code"
    assert np.array_equal(to_bf16_bits(-mid), want_mid | np.uint16(0x8000)), "negative midpoints"
    off = ulp * 2.0 ** -20                                      # 1/16 of a float32 unit at this scale
    assert np.array_equal(to_bf16_bits(mid + off), (k + 1).astype(np.uint16)), "just above a midpoint"
    assert np.array_equal(to_bf16_bits(mid - off), k), "just below a midpoint"
    assert np.array_equal(to_bf16_bits(lo), k), "representable values are kept"
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))
    assert np.array_equal(to_bf16_bits(x), reference(x)), "random values"
    assert np.array_equal(reference(mid), want_mid) and np.array_equal(reference(mid + off), (k + 1).astype(np.uint16))
