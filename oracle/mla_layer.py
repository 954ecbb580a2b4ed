"""CPU fp64 oracle for the steps on either side of the paged MLA decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests (and the benchmark's CPU baseline) do.  It
shares no code with the HIP library.

What is computed (plain definitions, float64 unless a step's output is an
encoding):

* Low-rank joint KV compression (FlashMLA-on-Ascend post, "MLA 的压缩原理", and
  its computation flow): keys and values of head h are up-projections of one
  shared latent row c_t, K_h = c W_UK[h], V_h = c W_UV[h].  In the absorbed form
  the decode runs on (the 576-wide rows of the FlashMLA-ETAP summary), the key
  up-projection is folded into the query and the value up-projection is applied
  after attention:
      q_latent[h] = W_UK[h] q_nope[h]          (W_UK[h]: 512 x 128)
      o[h]        = W_UV[h] out_latent[h]      (W_UV[h]: 128 x 512)
  so that q_latent . c = q_nope . (W_UK[h]^T c) and W_UV[h] (sum_t p_t c_t) =
  sum_t p_t (W_UV[h] c_t): the same attention as with decompressed per-head
  keys and values.  ``decompressed_attention`` evaluates that second form
  directly and pins the first.
* Rotary position embedding on the 64 rope columns of the query and of the new
  cache row (the rope part of the 576-wide row).  Reading taken (the pages do
  not spell it out): consecutive pairs (x[2i], x[2i+1]) rotate by the angle
  pos * base^(-2i/64), base 10000 by default.
* The new token's cache row: [c (512 latent), rope(k_pe, pos) (64)] stored at
  row pos % P of page block_table[b][pos // P]; in the fp8 layout the latent
  group g (columns 128g..128g+127) is stored as E4M3 codes of x / 2^e_g with
  e_g the smallest integer >= -126 such that max|x| <= 448 * 2^e_g (e_g = 0 for
  an all-zero group), rounded to nearest even, and the scale 2^e_g as float32.
  The lower limit keeps every scale a normal float32: a row's reader uses only
  the exponent field of a scale.

Weight layouts (this library's): W_UK as [H, 512, 128] (row e of head h maps
the 128 nope columns to latent column e), W_UV as [H, 128, 512].
"""
from __future__ import annotations

import numpy as np

from oracle.mla_oracle import decode_e4m3, widen_bf16

D_LATENT = 512
D_ROPE = 64
D_NOPE = 128
D_VOUT = 128
FP8_ROW_BYTES = 656


def rope(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate consecutive pairs of the last axis (64 wide) by pos * base^(-2i/64).
    x [..., 64] float64; pos broadcastable to x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    i = np.arange(D_ROPE // 2, dtype=np.float64)
    inv = np.power(float(base), -2.0 * i / D_ROPE)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def q_absorb(q_nope, q_pe, w_uk, positions, base: float = 10000.0):
    """q_nope [B, S, H, 128], q_pe [B, S, H, 64] (bf16 bits), w_uk [H, 512, 128] (bf16 bits),
    positions [B, S] -> query rows [B, S, H, 576] float64: [W_UK[h] q_nope, rope(q_pe, pos)]."""
    qn = widen_bf16(q_nope)
    w = widen_bf16(w_uk)
    lat = np.einsum("bshd,hed->bshe", qn, w)
    pe = rope(widen_bf16(q_pe), np.asarray(positions)[:, :, None], base)
    return np.concatenate([lat, pe], axis=-1)


def out_absorb(out_latent, w_uv):
    """out_latent [B, S, H, 512] float64 (already widened), w_uv [H, 128, 512] (bf16 bits)
    -> [B, S, H, 128] float64: o[h] = W_UV[h] out_latent[h]."""
    return np.einsum("bshe,hve->bshv", np.asarray(out_latent, dtype=np.float64), widen_bf16(w_uv))


def fp8_group_exponent(amax: float) -> int:
    """Smallest integer e >= -126 with amax <= 448 * 2^e (0 for amax == 0)."""
    if amax == 0.0:
        return 0
    if amax <= 448.0 * 2.0 ** -126:
        return -126
    e = int(np.ceil(np.log2(amax / 448.0)))
    while 448.0 * 2.0 ** (e - 1) >= amax:        # guard the log against rounding
        e -= 1
    while 448.0 * 2.0 ** e < amax:
        e += 1
    return e


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float64 values (|x| <= 448) to the nearest E4M3 code, ties to the even code;
    the sign bit is the sign of x (so tiny negative values give -0)."""
    x = np.asarray(x, dtype=np.float64)
    mag_vals = decode_e4m3(np.arange(0x7F, dtype=np.uint8))     # codes 0x00..0x7E, increasing
    a = np.abs(x)
    hi = np.clip(np.searchsorted(mag_vals, a), 1, 0x7E)
    lo = hi - 1
    dlo, dhi = a - mag_vals[lo], mag_vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= mag_vals[-1], 0x7E, pick)
    return (pick.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)).astype(np.uint8)


def cache_row(c_kv_bits, k_pe_bits, pos, kv_format: str = "bf16", base: float = 10000.0):
    """The stored row of one new token: bf16 [576] uint16, or fp8 [656] uint8."""
    pe = rope(widen_bf16(k_pe_bits), pos, base)
    pe_bits = _f64_to_bf16_bits(pe)
    if kv_format == "bf16":
        return np.concatenate([np.asarray(c_kv_bits, dtype=np.uint16), pe_bits])
    x = widen_bf16(c_kv_bits)
    row = np.zeros(FP8_ROW_BYTES, dtype=np.uint8)
    scales = np.zeros(4, dtype=np.float32)
    for g in range(4):
        grp = x[128 * g:128 * (g + 1)]
        e = fp8_group_exponent(float(np.max(np.abs(grp))))
        row[128 * g:128 * (g + 1)] = encode_e4m3(grp * 2.0 ** (-e))
        scales[g] = np.float32(2.0 ** e)
    row[512:640] = pe_bits.view(np.uint8)
    row[640:656] = scales.view(np.uint8)
    return row


def _f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, rounding the float64 value to nearest even at bf16 precision."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                            # x = m * 2^e, 0.5 <= |m| < 1
    q = np.round(m * 256.0)                       # 8 significant bits; np.round is ties-to-even
    y = (q / 256.0) * np.exp2(e.astype(np.float64))
    return (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def append_rows(kv_cache, block_table, c_kv, k_pe, positions, kv_format: str = "bf16", base: float = 10000.0):
    """A copy of kv_cache with the new tokens' rows written (c_kv [B, S, 512], k_pe [B, S, 64]
    bf16 bits; positions [B, S])."""
    kv = np.array(kv_cache, copy=True)
    P = kv.shape[1]
    B, S = np.asarray(positions).shape
    for b in range(B):
        for i in range(S):
            pos = int(positions[b, i])
            page = int(block_table[b, pos // P])
            kv[page, pos % P] = cache_row(c_kv[b, i], k_pe[b, i], pos, kv_format, base)
    return kv


def decompressed_attention(q_nope, q_pe, latent_rows, rope_rows, w_uk, w_uv, scale, positions, base=10000.0):
    """Attention written in the decompressed form, for one sequence: per head, keys
    K_h[t] = [W_UK[h]^T c_t, rope_t] and values V_h[t] = W_UV[h] c_t (float64).
    q_nope [S, H, 128], q_pe [S, H, 64] bits; latent_rows [L, 512], rope_rows [L, 64] float64
    (rope already applied, as stored).  Returns o [S, H, 128] float64."""
    qn = widen_bf16(q_nope)
    qp = rope(widen_bf16(q_pe), np.asarray(positions)[:, None], base)
    w_k = widen_bf16(w_uk)
    w_v = widen_bf16(w_uv)
    S, H = qn.shape[0], qn.shape[1]
    out = np.zeros((S, H, D_VOUT))
    for h in range(H):
        k_nope = latent_rows @ w_k[h]                        # [L, 128]
        v = latent_rows @ w_v[h].T                           # [L, 128]
        for i in range(S):
            s = scale * (k_nope @ qn[i, h] + rope_rows @ qp[i, h])
            p = np.exp(s - s.max())
            out[i, h] = (p / p.sum()) @ v
    return out
