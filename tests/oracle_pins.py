"""Pins that tie the fp64 oracle to facts other than itself.

Each pin takes the decode function under test (same signature as
``oracle.mla_oracle.decode``) and raises AssertionError when it disagrees with
what the mathematics or the pages fix.  ``test_oracle.py`` runs them on the
oracle; ``test_oracle_mutations.py`` runs them on copies of the oracle with a
planted mistake and requires every mistake to be caught by at least one pin.

Pins:
  decimal_brute_force   -- independent 40-digit decimal evaluation of the
                           definition (own bf16 decoding, own gather loop).
  single_token          -- L = 1: out is that token's V row, lse its score.
  equal_scores          -- latent half of q zero, identical rope rows:
                           out = mean of V rows, lse = s + ln L.
  shift_invariance      -- adding a vector to every rope row shifts all scores
                           of a row by the same constant: out unchanged, lse
                           shifted by scale * q_rope . delta (dyadic, exact in bf16).
  page_permutation      -- relabelling physical pages changes nothing.
  decomposition         -- two-token query == two one-token calls; 128 heads ==
                           8 slices of 16; a batch == separate sequences.
  sdpa_special_case     -- one contiguous page == torch SDPA in float64 on CPU.
  split_combine         -- results over disjoint token ranges merged by the
                           log-sum-exp rule equal the unsplit result.
  causal_*              -- the causal mask between query tokens (see below).
  fp8_*                 -- the FP8 cache rows: the E4M3 decoder against the
                           format's definition and torch's float8_e4m3fn, the
                           exponent-only group scales, a decimal brute force on
                           fp8 rows, and fp8 rows against a bf16 cache holding
                           the same values.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np

from mla_decode_attention_paged_amd import inputs as gen

D_QK, D_V = 576, 512
TOL = 1e-12


# ----------------------------------------------------------------------------- decimal
def _bf16_to_decimal(bits: int) -> Decimal:
    """Decode a bf16 bit pattern by its fields (sign, 8-bit exponent, 7-bit fraction)."""
    bits = int(bits)
    sign = -1 if bits >> 15 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    with localcontext() as ctx:
        ctx.prec = 200                                  # enough digits to hold any bf16 exactly
        if exp == 0:
            v = Decimal(man) / Decimal(128) * (Decimal(2) ** -126)
        elif exp == 0xFF:
            raise ValueError("non-finite bf16 in decimal brute force")
        else:
            v = (Decimal(128 + man) / Decimal(128)) * (Decimal(2) ** (exp - 127))
        return sign * v


def _e4m3_to_decimal(code: int) -> Decimal:
    """Decode an OCP E4M3 byte by its fields (sign, 4-bit exponent bias 7, 3-bit mantissa)."""
    code = int(code)
    if code & 0x7F == 0x7F:
        raise ValueError("NaN E4M3 code in decimal brute force")
    sign = -1 if code >> 7 else 1
    exp = (code >> 3) & 0xF
    man = code & 7
    with localcontext() as ctx:
        ctx.prec = 60
        if exp == 0:
            v = Decimal(man) * (Decimal(2) ** -9)
        else:
            v = (Decimal(8 + man) / Decimal(8)) * (Decimal(2) ** (exp - 7))
        return sign * v


def _decimal_row(row) -> list:
    """One cache row as 576 Decimals: bf16 [576] uint16, or an fp8 row [656] uint8."""
    row = np.asarray(row)
    if row.dtype != np.uint8:
        return [_bf16_to_decimal(x) for x in row.tolist()]
    b = [int(x) for x in row.tolist()]
    factors = []
    for g in range(4):
        word = b[640 + 4 * g] | (b[641 + 4 * g] << 8) | (b[642 + 4 * g] << 16) | (b[643 + 4 * g] << 24)
        factors.append(Decimal(2) ** (((word >> 23) & 0xFF) - 127))
    latent = [_e4m3_to_decimal(b[c]) * factors[c // 128] for c in range(512)]
    rope = [_bf16_to_decimal(b[512 + 2 * j] | (b[513 + 2 * j] << 8)) for j in range(64)]
    return latent + rope


def decimal_decode(q, kv, block_table, seqlens, scale, page_size, rows=None, causal=False):
    """Brute-force paged MLA decode at 40 significant digits. Returns nested lists.
    causal: query token i of S_q sees tokens t <= L - S_q + i."""
    results = {}
    with localcontext() as ctx:
        ctx.prec = 40
        sc = Decimal(float(np.float32(scale)))
        B, S, H = q.shape[0], q.shape[1], q.shape[2]
        for b in range(B):
            L = int(seqlens[b])
            keys = []
            for t in range(L):
                page = int(block_table[b][t // page_size])
                keys.append(_decimal_row(kv[page][t % page_size]))
            for i in range(S):
                for h in range(H):
                    if rows is not None and (b, i, h) not in rows:
                        continue
                    qv = [_bf16_to_decimal(x) for x in q[b, i, h].tolist()]
                    vis = keys if not causal else keys[:max(0, L - S + i + 1)]
                    if not vis:
                        results[(b, i, h)] = ([0.0] * D_V, float("-inf"))
                        continue
                    s = [sc * sum(qd * kd for qd, kd in zip(qv, k)) for k in vis]
                    m = max(s)
                    z = sum((st - m).exp() for st in s)
                    lse = m + z.ln()
                    w = [(st - lse).exp() for st in s]
                    out = [sum(w[t] * vis[t][d] for t in range(len(vis))) for d in range(D_V)]
                    results[(b, i, h)] = ([float(x) for x in out], float(lse))
    return results


def decimal_brute_force(decode_fn, cases=None):
    if cases is None:
        cases = [
            dict(batch=2, q_len=1, num_heads=2, page_size=16, lengths=[1, 17], seed=11),
            dict(batch=2, q_len=2, num_heads=2, page_size=16, lengths=[3, 5], seed=12),
            dict(batch=2, q_len=1, num_heads=16, page_size=64, lengths=[2, 65], seed=13),
            dict(batch=2, q_len=2, num_heads=16, page_size=64, lengths=[64, 1], seed=14),
        ]
    worst = 0.0
    for c in cases:
        p = gen.make_problem(**c)
        out, lse = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, p.page_size)
        rng = np.random.default_rng(c["seed"])
        # every row for tiny head counts; a few sampled rows for 16 heads
        rows = None
        if p.num_heads > 4:
            rows = {(b, int(rng.integers(p.q_len)), int(rng.integers(p.num_heads))) for b in range(p.batch)}
            rows |= {(b, p.q_len - 1, p.num_heads - 1) for b in range(p.batch)}
        ref = decimal_decode(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale,
                             p.page_size, rows)
        for (b, i, h), (o_ref, l_ref) in ref.items():
            eo = float(np.max(np.abs(np.asarray(out[b, i, h]) - np.asarray(o_ref))))
            el = abs(float(lse[b, i, h]) - l_ref)
            worst = max(worst, eo, el)
            assert eo <= TOL and el <= TOL, f"decimal brute force: case {c} row {(b, i, h)} out err {eo} lse err {el}"
    return worst


# ----------------------------------------------------------------------------- closed forms
def single_token(decode_fn):
    p = gen.make_problem(batch=3, q_len=2, num_heads=16, page_size=16, lengths=[1, 1, 1], seed=21,
                         extra_pages=2)
    out, lse = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, p.page_size)
    for b in range(p.batch):
        row = p.kv_cache[p.block_table[b, 0], 0]
        v = gen.bf16_bits_to_f32(row[:D_V]).astype(np.float64)
        k = gen.bf16_bits_to_f32(row).astype(np.float64)
        for i in range(p.q_len):
            for h in range(p.num_heads):
                assert np.array_equal(out[b, i, h], v), "single token: out != that token's V row"
                qv = gen.bf16_bits_to_f32(p.q[b, i, h]).astype(np.float64)
                s0 = math.fsum((p.softmax_scale * qv * k).tolist())
                assert abs(lse[b, i, h] - s0) <= TOL * max(1.0, abs(s0)), "single token: lse != score"


def equal_scores(decode_fn):
    rng = np.random.default_rng(31)
    L, P = 77, 16
    p = gen.make_problem(batch=2, q_len=1, num_heads=16, page_size=P, lengths=[L, 40], seed=31)
    q = p.q.copy()
    q[..., :D_V] = 0                                    # scores depend on the rope part only
    kv = p.kv_cache.copy()
    rope = gen.f32_to_bf16_bits(rng.standard_normal(D_QK - D_V).astype(np.float32))
    kv[..., D_V:] = rope                                # identical rope part in every row
    out, lse = decode_fn(q, kv, p.block_table, p.cache_seqlens, p.softmax_scale, P)
    for b in range(p.batch):
        Lb = int(p.cache_seqlens[b])
        t = np.arange(Lb)
        rows = kv[p.block_table[b, t // P], t % P]
        mean_v = gen.bf16_bits_to_f32(rows[:, :D_V]).astype(np.float64).mean(axis=0)
        rr = gen.bf16_bits_to_f32(rope).astype(np.float64)
        for h in range(p.num_heads):
            qr = gen.bf16_bits_to_f32(q[b, 0, h, D_V:]).astype(np.float64)
            s = p.softmax_scale * math.fsum((qr * rr).tolist())
            assert np.max(np.abs(out[b, 0, h] - mean_v)) <= TOL, "equal scores: out != mean of V"
            assert abs(lse[b, 0, h] - (s + math.log(Lb))) <= TOL, "equal scores: lse != s + ln L"


def _dyadic_bf16(rng, shape, lo=-32, hi=32, den=16):
    return gen.f32_to_bf16_bits((rng.integers(lo, hi, size=shape) / den).astype(np.float32))


def shift_invariance(decode_fn):
    rng = np.random.default_rng(41)
    P = 16
    p = gen.make_problem(batch=2, q_len=2, num_heads=16, page_size=P, lengths=[50, 33], seed=41)
    kv = _dyadic_bf16(rng, p.kv_cache.shape)            # entries k/16 in [-2, 2)
    q = _dyadic_bf16(rng, p.q.shape)
    delta = rng.integers(-4, 5, size=D_QK - D_V).astype(np.float32)
    kv2 = kv.copy()
    shifted = gen.bf16_bits_to_f32(kv[..., D_V:]) + delta
    kv2[..., D_V:] = gen.f32_to_bf16_bits(shifted)
    assert np.array_equal(gen.bf16_bits_to_f32(kv2[..., D_V:]), shifted), "shift not exact in bf16"
    o1, l1 = decode_fn(q, kv, p.block_table, p.cache_seqlens, p.softmax_scale, P)
    o2, l2 = decode_fn(q, kv2, p.block_table, p.cache_seqlens, p.softmax_scale, P)
    # V (latent columns) is untouched, so only the scores move, all by the same amount per row
    assert np.max(np.abs(o1 - o2)) <= TOL, "shift invariance: out changed"
    qr = gen.bf16_bits_to_f32(q[..., D_V:]).astype(np.float64)
    expect = l1 + p.softmax_scale * (qr @ delta.astype(np.float64))
    assert np.max(np.abs(l2 - expect)) <= 1e-11, "shift invariance: lse shift wrong"


def page_permutation(decode_fn):
    rng = np.random.default_rng(51)
    P = 16
    p = gen.make_problem(batch=3, q_len=1, num_heads=16, page_size=P, lengths=[70, 16, 33], seed=51,
                         extra_pages=3)
    o1, l1 = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, P)
    perm = rng.permutation(p.num_pages)                 # new physical slot of each page
    kv2 = np.empty_like(p.kv_cache)
    kv2[perm] = p.kv_cache
    bt2 = np.where(p.block_table >= 0, perm[np.maximum(p.block_table, 0)], -1).astype(np.int32)
    o2, l2 = decode_fn(p.q, kv2, bt2, p.cache_seqlens, p.softmax_scale, P)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "page permutation changed the result"


def decomposition(decode_fn):
    P = 16
    # two-token query == two one-token queries
    p = gen.make_problem(batch=2, q_len=2, num_heads=16, page_size=P, lengths=[45, 29], seed=61)
    o, l = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, P)
    for i in range(2):
        oi, li = decode_fn(np.ascontiguousarray(p.q[:, i:i + 1]), p.kv_cache, p.block_table,
                           p.cache_seqlens, p.softmax_scale, P)
        assert np.max(np.abs(oi[:, 0] - o[:, i])) <= TOL and np.max(np.abs(li[:, 0] - l[:, i])) <= TOL, \
            "decomposition: q_len 2 != two q_len 1 calls"
    # 128 heads == 8 slices of 16
    p = gen.make_problem(batch=1, q_len=1, num_heads=128, page_size=P, lengths=[37], seed=62)
    o, l = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, P)
    for s in range(8):
        sl = slice(16 * s, 16 * s + 16)
        os_, ls_ = decode_fn(np.ascontiguousarray(p.q[:, :, sl]), p.kv_cache, p.block_table,
                             p.cache_seqlens, p.softmax_scale, P)
        assert np.max(np.abs(os_ - o[:, :, sl])) <= TOL and np.max(np.abs(ls_ - l[:, :, sl])) <= TOL, \
            "decomposition: 128 heads != 8 x 16"
    # a batch == separate sequences
    p = gen.make_problem(batch=3, q_len=1, num_heads=16, page_size=P, lengths=[20, 51, 3], seed=63)
    o, l = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, P)
    for b in range(3):
        ob, lb = decode_fn(p.q[b:b + 1], p.kv_cache, p.block_table[b:b + 1], p.cache_seqlens[b:b + 1],
                           p.softmax_scale, P)
        assert np.max(np.abs(ob[0] - o[b])) <= TOL and np.max(np.abs(lb[0] - l[b])) <= TOL, \
            "decomposition: batch != separate sequences"


def sdpa_special_case(decode_fn):
    import torch
    L = 96
    p = gen.make_problem(batch=1, q_len=2, num_heads=16, page_size=L, lengths=[L], seed=71)
    o, l = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, L)
    k = torch.from_numpy(gen.bf16_bits_to_f32(p.kv_cache[0]).astype(np.float64))       # [L, 576]
    q = torch.from_numpy(gen.bf16_bits_to_f32(p.q[0]).astype(np.float64))             # [2, 16, 576]
    qh = q.permute(1, 0, 2).unsqueeze(0)                                                # [1, H, 2, 576]
    kh = k.unsqueeze(0).unsqueeze(0).expand(1, 16, L, D_QK).contiguous()
    vh = k[:, :D_V].unsqueeze(0).unsqueeze(0).expand(1, 16, L, D_V).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, scale=p.softmax_scale)
    ref = ref[0].permute(1, 0, 2).numpy()                                               # [2, 16, 512]
    ref_lse = torch.logsumexp(p.softmax_scale * (qh @ kh.transpose(-1, -2)), dim=-1)[0].T.numpy()
    assert np.max(np.abs(o[0] - ref)) <= TOL, "SDPA special case: out"
    assert np.max(np.abs(l[0] - ref_lse)) <= TOL, "SDPA special case: lse"


def split_combine(attend_fn, combine_fn):
    rng = np.random.default_rng(81)
    L = 200
    k = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal((L, D_QK), dtype=np.float32))).astype(np.float64)
    q = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal((16, D_QK), dtype=np.float32))).astype(np.float64)
    sc = gen.SOFTMAX_SCALE
    o_ref, l_ref = attend_fn(q, k, k[:, :D_V], sc)
    for cuts in ([1], [64, 128], [3, 4, 5, 199], list(range(16, 200, 16))):
        bounds = [0] + cuts + [L]
        outs, lses = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            o, l = attend_fn(q, k[a:b], k[a:b, :D_V], sc)
            outs.append(o)
            lses.append(l)
        # an empty part must not change anything
        o0, l0 = attend_fn(q, k[:0], k[:0, :D_V], sc)
        outs.append(o0)
        lses.append(l0)
        o, l = combine_fn(np.stack(outs), np.stack(lses))
        assert np.max(np.abs(o - o_ref)) <= TOL and np.max(np.abs(l - l_ref)) <= TOL, f"split/combine at {cuts}"




def causal_decimal(decode_fn):
    """Causal two-token queries against the decimal brute force (including L = 1, where
    the first query token sees nothing)."""
    for c in (dict(batch=3, q_len=2, num_heads=2, page_size=16, lengths=[1, 2, 18], seed=91),
              dict(batch=1, q_len=3, num_heads=2, page_size=16, lengths=[5], seed=92)):
        p = gen.make_problem(**c)
        out, lse = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, p.page_size,
                             causal=True)
        ref = decimal_decode(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, p.page_size,
                             causal=True)
        for (b, i, h), (o_ref, l_ref) in ref.items():
            if l_ref == float("-inf"):
                assert np.all(out[b, i, h] == 0) and lse[b, i, h] == -np.inf, "causal: empty row"
                continue
            assert np.max(np.abs(out[b, i, h] - np.asarray(o_ref))) <= TOL and abs(lse[b, i, h] - l_ref) <= TOL


def causal_decomposition(decode_fn):
    """Causal query token i of S_q == a one-token query over the first L - S_q + i + 1 tokens."""
    P = 16
    p = gen.make_problem(batch=3, q_len=2, num_heads=16, page_size=P, lengths=[40, 17, 2], seed=93)
    o, l = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, P, causal=True)
    for i in range(2):
        lens = np.maximum(p.cache_seqlens - 2 + i + 1, 0).astype(np.int32)
        oi, li = decode_fn(np.ascontiguousarray(p.q[:, i:i + 1]), p.kv_cache, p.block_table, lens,
                           p.softmax_scale, P)
        assert np.max(np.abs(oi[:, 0] - o[:, i])) <= TOL and np.max(np.abs(li[:, 0] - l[:, i])) <= TOL
    # and the last query token sees everything: same as the unmasked call
    o2, l2 = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, P)
    assert np.max(np.abs(o2[:, 1] - o[:, 1])) <= TOL
    assert np.max(np.abs(o2[:, 0] - o[:, 0])) > 1e-6, "mask had no effect"


ALL_DECODE_PINS = [decimal_brute_force, single_token, equal_scores, shift_invariance, page_permutation,
                   decomposition, sdpa_special_case, causal_decimal, causal_decomposition]


# ----------------------------------------------------------------------------- fp8 cache rows
def fp8_decoder_spec_values(decode_e4m3):
    """E4M3 values fixed by the format: zero, signed zero, the smallest subnormal, the
    largest subnormal, the smallest normal, one, the largest finite value, NaN."""
    codes = np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0xB8, 0x7E, 0xFE, 0x7F, 0xFF, 0x3F], dtype=np.uint8)
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, -1.0, 448.0, -448.0, np.nan, np.nan, 1.875]
    got = decode_e4m3(codes)
    for c, g, w in zip(codes, got, want):
        if np.isnan(w):
            assert np.isnan(g), f"code {c:#x}: {g} is not NaN"
        else:
            assert g == w and np.signbit(g) == np.signbit(w), f"code {c:#x}: {g} != {w}"


def fp8_decoder_matches_torch(decode_e4m3):
    """All 256 codes against torch's float8_e4m3fn (a library that implements the same format)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(ref)], ref[~np.isnan(ref)])


def _fp8_row(latent_codes, rope_bits, scales):
    row = np.zeros(656, dtype=np.uint8)
    row[:512] = latent_codes
    row[512:640] = np.asarray(rope_bits, dtype=np.uint16).view(np.uint8)
    row[640:656] = np.asarray(scales, dtype=np.float32).view(np.uint8)
    return row


def fp8_scale_exponent_only(widen_fp8_rows):
    """A group scale counts only through its exponent: 1.5 acts as 1, 0.3 as 0.25, 96 as 64.
    Group g covers latent columns [128g, 128g + 128); rope columns are never scaled."""
    codes = np.full(512, 0x38, dtype=np.uint8)           # every latent value 1.0
    rope = gen.f32_to_bf16_bits(np.linspace(-2, 2, 64).astype(np.float32))
    w = widen_fp8_rows(_fp8_row(codes, rope, [1.5, 0.3, 96.0, 2.0 ** -20])[None])[0]
    for g, f in enumerate([1.0, 0.25, 64.0, 2.0 ** -20]):
        assert np.all(w[128 * g:128 * (g + 1)] == f), f"group {g}"
    assert np.array_equal(w[512:], gen.bf16_bits_to_f32(rope).astype(np.float64))


def fp8_decimal_brute_force(decode_fn):
    cases = [dict(batch=2, q_len=1, num_heads=2, page_size=16, lengths=[1, 19], seed=41, kv_format="fp8"),
             dict(batch=1, q_len=2, num_heads=2, page_size=16, lengths=[6], seed=42, kv_format="fp8")]
    for c in cases:
        p = gen.make_problem(**c)
        out, lse = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, p.page_size)
        ref = decimal_decode(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, p.page_size)
        for (b, i, h), (o_ref, l_ref) in ref.items():
            eo = float(np.max(np.abs(np.asarray(out[b, i, h]) - np.asarray(o_ref))))
            el = abs(float(lse[b, i, h]) - l_ref)
            assert eo <= TOL and el <= TOL, f"fp8 decimal brute force: {c} row {(b, i, h)}: {eo} {el}"


def fp8_matches_bf16_cache(decode_fn):
    """fp8 rows whose values are exact in bf16 (they all are: 4 significant bits times a power
    of two) give the same result as a bf16 cache that stores those values."""
    p = gen.make_problem(batch=3, q_len=2, num_heads=16, page_size=16, lengths=[33, 1, 70], seed=43,
                         kv_format="fp8")
    rows = p.kv_cache.reshape(-1, 656)
    bf = np.empty((rows.shape[0], D_QK), dtype=np.uint16)
    for r in range(rows.shape[0]):
        bf[r] = [int(x) for x in (np.array([float(v) for v in _decimal_row(rows[r])], dtype=np.float32)
                                  .view(np.uint32) >> 16)]
    kv_bf = bf.reshape(p.kv_cache.shape[0], p.kv_cache.shape[1], D_QK)
    o8, l8 = decode_fn(p.q, p.kv_cache, p.block_table, p.cache_seqlens, p.softmax_scale, p.page_size)
    ob, lb = decode_fn(p.q, kv_bf, p.block_table, p.cache_seqlens, p.softmax_scale, p.page_size)
    assert np.max(np.abs(o8 - ob)) <= TOL and np.max(np.abs(l8 - lb)) <= TOL


FP8_DECODE_PINS = [fp8_decimal_brute_force, fp8_matches_bf16_cache]
ALL_DECODE_PINS = ALL_DECODE_PINS + FP8_DECODE_PINS
