"""CPU fp64 oracle for absorbed MLA decode over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package smoke check and the CPU
baseline leg of the benchmark do.  It shares no code with the HIP library; the
only thing both sides consume is the seeded input arrays.

What is computed (plain definitions, written out; every float op in float64):

* Standard attention, S = Q K^T, P = softmax(S), O = P V  -- FlashMLA-ETAP
  summary (gist.science), "Core mechanism" (核心机制).  The transposed pipeline
  on that page (S^T = K Q^T, P^T = softmax(S^T), O = (V^T P^T)^T) is the same
  mathematics, so the oracle uses the untransposed definition.
* Absorbed MLA: one 576-wide cached row per token, shared by every query head
  (the low-rank joint compression of the same page's "Implementation details"
  and the 16-head, 576-dim configuration of its "Limitations noted by the
  authors").  Scores use all 576 columns; V is the first 512 columns of the
  same row (512 latent + 64 rope).
* Paged cache: token t of sequence b lives in physical page
  block_table[b][t // page_size], row t % page_size (PagedAttention, listed
  under "Builds on" on the mlsanity.com page of the same paper).
* Split-and-merge of partial results (log-sum-exp weighting).  The pages give
  the streaming (online) form of softmax -- juejin.cn FlashMLA explainer,
  section 三 "在线 Softmax"; FlashMLA-on-Ascend post, "FlashMLA 的计算流程" step
  4 -- whose exact consequence is that softmax over a union of token ranges
  equals the LSE-weighted sum of the per-range results; ``combine`` states that
  identity directly.

* FP8 latent cache (a cache format the pages name for FlashMLA without fixing
  it; the layout is this library's): each token row is 656 bytes -- 512 OCP
  FP8 E4M3 codes for the latent columns, 64 bf16 rope columns, and four float32
  group scales of which only the exponent counts.  ``widen_fp8_rows`` decodes a
  row from the E4M3 definition (sign, 4-bit exponent with bias 7, 3-bit mantissa,
  subnormals at exponent 0, S.1111.111 is NaN, no infinities) and multiplies
  latent column c by 2^(E - 127), E the biased exponent of scale c // 128.

Readings where the pages are silent (each is listed in the design notes):
  - lse is the natural log of sum_t exp(s_t) with s_t = scale * q . k_t;
  - an empty context (L = 0) gives out = 0 and lse = -inf;
  - by default both query tokens of a two-token query see all L cached tokens
    (no mask); with ``causal=True`` query token i of S_q sits at position
    L - S_q + i and sees tokens t <= L - S_q + i (the S_q new tokens' rows are
    already in the cache, as for speculative / multi-token decode);
  - rows past L and unmapped block_table entries are never read.
"""
from __future__ import annotations

import numpy as np

D_QK = 576
D_V = 512


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of float32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


FP8_ROW_BYTES = 656


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64, exactly."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def widen_fp8_rows(rows: np.ndarray) -> np.ndarray:
    """fp8 cache rows [L, 656] uint8 -> float64 [L, 576] (latent decoded and scaled, rope widened)."""
    r = np.asarray(rows, dtype=np.uint8)
    L = r.shape[0]
    # every code decoded once by the definition above, then looked up (the same values)
    latent = decode_e4m3(np.arange(256, dtype=np.uint8))[r[:, :D_V]]
    scale_bits = np.ascontiguousarray(r[:, 640:656]).view(np.uint32).reshape(L, 4)
    factor = np.exp2(((scale_bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.float64) - 127.0)
    latent = latent * np.repeat(factor, D_V // 4, axis=1)
    rope = widen_bf16(np.ascontiguousarray(r[:, D_V:640]).view(np.uint16).reshape(L, D_QK - D_V))
    return np.concatenate([latent, rope], axis=1)


def widen_rows(rows: np.ndarray) -> np.ndarray:
    """Cache rows as stored (bf16 [L, 576] uint16 or fp8 [L, 656] uint8) -> float64 [L, 576]."""
    if np.asarray(rows).dtype == np.uint8:
        return widen_fp8_rows(rows)
    return widen_bf16(rows)


def gather_sequence(kv_cache: np.ndarray, block_table_row: np.ndarray, length: int,
                    page_size: int) -> np.ndarray:
    """Logical rows 0..length-1 of one sequence, in token order, as stored (uint16 bits).

    Token t -> page block_table_row[t // page_size], row t % page_size.
    """
    t = np.arange(int(length), dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // page_size]
    return np.asarray(kv_cache)[pages, t % page_size]


def attend(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float):
    """Softmax attention of R query rows over L key/value rows, float64.

    Returns (out [R, Dv], lse [R]) with
        s[r, t] = scale * sum_d q[r, d] k[t, d]
        lse[r]  = log sum_t exp(s[r, t])            (computed as m + log sum exp(s - m))
        out[r]  = sum_t exp(s[r, t] - lse[r]) v[t]
    """
    q = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    v = np.asarray(v_rows, dtype=np.float64)
    R, L = q.shape[0], k.shape[0]
    if L == 0:
        return np.zeros((R, v.shape[1])), np.full(R, -np.inf)
    s = float(scale) * (q @ k.T)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p @ v, lse


def decode_sequence(q_b: np.ndarray, kv_cache: np.ndarray, block_table_row: np.ndarray,
                    length: int, softmax_scale: float, page_size: int, causal: bool = False):
    """One sequence: q_b [S_q, H, 576] bits -> (out [S_q, H, 512], lse [S_q, H]) float64."""
    s_q, h = q_b.shape[0], q_b.shape[1]
    rows = gather_sequence(kv_cache, block_table_row, length, page_size)
    k = widen_rows(rows)
    if not causal:
        q = widen_bf16(q_b).reshape(s_q * h, D_QK)
        out, lse = attend(q, k, k[:, :D_V], softmax_scale)
        return out.reshape(s_q, h, D_V), lse.reshape(s_q, h)
    out = np.empty((s_q, h, D_V))
    lse = np.empty((s_q, h))
    for i in range(s_q):
        visible = max(0, int(length) - s_q + i + 1)       # tokens t <= L - S_q + i
        out[i], lse[i] = attend(widen_bf16(q_b[i]), k[:visible], k[:visible, :D_V], softmax_scale)
    return out, lse


def decode(q: np.ndarray, kv_cache: np.ndarray, block_table: np.ndarray,
           cache_seqlens: np.ndarray, softmax_scale: float, page_size: int,
           batch_indices=None, causal: bool = False):
    """Paged MLA decode for every (or the listed) sequence.

    q [B, S_q, H, 576] bf16 bits; kv_cache [num_pages, page_size, 576] bf16 bits or
    [num_pages, page_size, 656] uint8 fp8 rows;
    block_table [B, max_pages] int32; cache_seqlens [B] int32.
    Returns out [B, S_q, H, 512] and lse [B, S_q, H] in float64 (rows of
    sequences not listed in ``batch_indices`` are left NaN).
    """
    B, s_q, h = q.shape[0], q.shape[1], q.shape[2]
    out = np.full((B, s_q, h, D_V), np.nan)
    lse = np.full((B, s_q, h), np.nan)
    idx = range(B) if batch_indices is None else batch_indices
    for b in idx:
        out[b], lse[b] = decode_sequence(q[b], kv_cache, block_table[b], int(cache_seqlens[b]),
                                         softmax_scale, page_size, causal)
    return out, lse


def combine(partial_out: np.ndarray, partial_lse: np.ndarray):
    """Merge results computed over disjoint token ranges of the same rows.

    partial_out [S, R, Dv], partial_lse [S, R] (each part normalised over its own
    range).  Returns (out [R, Dv], lse [R]):
        lse = M + log sum_s exp(lse_s - M),   M = max_s lse_s
        out = sum_s exp(lse_s - lse) out_s
    Parts with lse_s = -inf (empty ranges) get weight 0.
    """
    po = np.asarray(partial_out, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    M = pl.max(axis=0)
    safe_M = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(pl - safe_M[None, :])
    tot = w.sum(axis=0)
    lse = np.where(np.isfinite(M), safe_M + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    wn = np.where(tot[None, :] > 0, w / np.where(tot > 0, tot, 1.0)[None, :], 0.0)
    out = np.einsum("sr,srd->rd", wn, po)
    return out, lse


def split_attend(q_rows, k_rows, v_rows, scale, cuts):
    """attend() over the token ranges between consecutive ``cuts``, merged by combine()."""
    bounds = [0] + sorted(int(c) for c in cuts) + [k_rows.shape[0]]
    outs, lses = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, l = attend(q_rows, k_rows[a:b], v_rows[a:b], scale)
        outs.append(o)
        lses.append(l)
    return combine(np.stack(outs), np.stack(lses))
