"""Seeded synthetic inputs for paged MLA decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the GPU path (through the package binding) and the
CPU oracle (under ``oracle/``) consume what it produces.

Workload shape (DeepSeek-R1 decode as measured on the FlashMLA-ETAP pages:
16 heads per GPU, 576-wide heads, batch 16/32, context up to 64K, query of 1-2
tokens -- FlashMLA-ETAP summary, "Problem statement" and "Experimental
results"; 576 = 512 latent + 64 rope).  Cache rows and queries are N(0,1)
float32 draws rounded to bf16 (round-to-nearest-even); bf16 values are carried
as ``uint16`` bit patterns.

Draw order for one problem (fixed so that a seed names one input set):
  1. ragged lengths (only when ``lengths`` is not given),
  2. the page permutation,
  3. the cache values (page by page, in physical order),
  4. the query values.

FP8 cache rows (``kv_format="fp8"``), 656 bytes per token:
  bytes [0, 512)    latent columns 0..511 as OCP FP8 E4M3 codes,
  bytes [512, 640)  rope columns 512..575 as bf16,
  bytes [640, 656)  four float32 group scales, one per 128 latent columns; only
                    the exponent counts (a column's value is its code's value times
                    2^(biased exponent - 127) of its group's scale).
The generator draws N(0,1) float32 latent values, picks per (row, group) the
power of two 2^ceil(log2(max|x| / 448)) as the scale and lets torch round x /
scale to E4M3 (an input encoding; the decode never encodes).  Rope columns are
N(0,1) rounded to bf16.  Step 3 then draws all latent values (row chunks), then
all rope values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

D_QK = 576          # latent (512) + rope (64)
D_V = 512           # latent columns, which double as V
SOFTMAX_SCALE = float(np.float32(1.0 / math.sqrt(192.0)))

_CHUNK = 1 << 24    # elements generated per RNG call (bounds host memory)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even) and return the uint16 bit pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)
FP8_ROW_BYTES = 656         # 512 E4M3 latent + 64 bf16 rope + 4 float32 group scales
FP8_NAN = np.uint8(0x7F)
FP8_GROUP = 128             # latent columns per scale
_ROW_CHUNK = 32768          # fp8 rows generated per RNG call


@dataclass
class Problem:
    """One decode call's inputs, host side."""
    q: np.ndarray              # [B, S_q, H, 576] uint16 (bf16 bits)
    kv_cache: np.ndarray       # [num_pages, P, 576] uint16 (bf16 bits) or [num_pages, P, 656] uint8 (fp8 rows)
    block_table: np.ndarray    # [B, max_pages_per_seq] int32, -1 where unused
    cache_seqlens: np.ndarray  # [B] int32
    softmax_scale: float
    page_size: int
    out_fp32: bool = False
    seed: int = 0
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_len(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_pages(self) -> int:
        return int(self.kv_cache.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def kv_format(self) -> str:
        return "fp8" if self.kv_cache.dtype == np.uint8 else "bf16"


def _normal_bf16(rng: np.random.Generator, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out


def _fp8_rows(rng: np.random.Generator, n: int) -> np.ndarray:
    """n cache rows in the fp8 layout (see the module docstring)."""
    import torch
    rows = np.empty((n, FP8_ROW_BYTES), dtype=np.uint8)
    for s in range(0, n, _ROW_CHUNK):
        e = min(n, s + _ROW_CHUNK)
        x = rng.standard_normal((e - s, D_V), dtype=np.float32).reshape(e - s, D_V // FP8_GROUP, FP8_GROUP)
        amax = np.maximum(np.abs(x).max(axis=2), np.float32(2.0 ** -100))
        scale = np.exp2(np.ceil(np.log2(amax.astype(np.float64) / 448.0))).astype(np.float32)
        codes = torch.from_numpy(np.ascontiguousarray(x / scale[:, :, None])).to(torch.float8_e4m3fn)
        rows[s:e, :D_V] = codes.view(torch.uint8).numpy().reshape(e - s, D_V)
        rows[s:e, 640:656] = scale.view(np.uint8).reshape(e - s, 16)
    for s in range(0, n, _ROW_CHUNK):
        e = min(n, s + _ROW_CHUNK)
        rope = f32_to_bf16_bits(rng.standard_normal((e - s, D_QK - D_V), dtype=np.float32))
        rows[s:e, D_V:640] = rope.view(np.uint8).reshape(e - s, 128)
    return rows


def draw_layout(rng: np.random.Generator, batch: int, page_size: int, lengths=None, ragged_range=None,
                extra_pages: int = 0, identity_pages: bool = False):
    """Steps 1 and 2 of the draw order: the context lengths (drawn only when not given) and the
    page table.  Returns (lengths int32 [B], block_table int32 [B, max_pages], num_pages)."""
    if lengths is None:
        lo, hi = ragged_range
        lengths = rng.integers(lo, hi, endpoint=True, size=batch)
    lengths = np.broadcast_to(np.asarray(lengths, dtype=np.int64), (batch,)).astype(np.int32)
    pages_per = [(int(L) + page_size - 1) // page_size for L in lengths]
    used = int(sum(pages_per))
    num_pages = used + int(extra_pages)
    max_pages = max(1, max(pages_per) if pages_per else 1)
    perm = np.arange(num_pages) if identity_pages else rng.permutation(num_pages)
    block_table = np.full((batch, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per):
        block_table[b, :n] = perm[off:off + n]
        off += n
    return lengths, block_table, num_pages


def config_layout(name: str, seed=None):
    """The named workload's lengths and page table (its recipe's steps 1 and 2) and its shape:
    (lengths, block_table, num_pages, dict of the config's other fields, seed)."""
    cfg = dict(CONFIGS[name])
    if seed is None:
        seed = CONFIG_ORDER.index(name)
    rng = np.random.default_rng(seed)
    lengths, block_table, num_pages = draw_layout(rng, cfg["batch"], cfg["page_size"], cfg.get("lengths"),
                                                  cfg.get("ragged_range"))
    return lengths, block_table, num_pages, cfg, seed


def make_problem(batch: int, q_len: int, num_heads: int, page_size: int,
                 lengths=None, *, seed: int = 0, ragged_range=None,
                 out_fp32: bool = False, tail: str = "normal",
                 extra_pages: int = 0, softmax_scale: float = SOFTMAX_SCALE,
                 identity_pages: bool = False, name: str = "", kv_format: str = "bf16") -> Problem:
    """Draw one paged decode problem.

    lengths        -- per-sequence context lengths (int or sequence); if None,
                      drawn uniformly from ``ragged_range`` (inclusive).
    tail           -- "normal": rows past a sequence's end in its last page hold
                      N(0,1) values; "nan": they (and the extra pages) hold NaN.
    extra_pages    -- physical pages that no sequence maps (filled like the tail).
    identity_pages -- block_table maps pages in order (no permutation draw).
    """
    rng = np.random.default_rng(seed)
    lengths, block_table, num_pages = draw_layout(rng, batch, page_size, lengths, ragged_range, extra_pages,
                                                  identity_pages)
    if kv_format == "bf16":
        kv = _normal_bf16(rng, num_pages * page_size * D_QK).reshape(num_pages, page_size, D_QK)
    elif kv_format == "fp8":
        kv = _fp8_rows(rng, num_pages * page_size).reshape(num_pages, page_size, FP8_ROW_BYTES)
    else:
        raise ValueError(f"unknown kv_format {kv_format!r}")
    q = _normal_bf16(rng, batch * q_len * num_heads * D_QK).reshape(batch, q_len, num_heads, D_QK)
    if tail == "nan":
        poison_unused(kv, block_table, lengths, page_size)
    elif tail != "normal":
        raise ValueError(f"unknown tail mode {tail!r}")
    return Problem(q=q, kv_cache=kv, block_table=block_table, cache_seqlens=lengths,
                   softmax_scale=float(softmax_scale), page_size=page_size, out_fp32=out_fp32,
                   seed=seed, name=name)


def poison_unused(kv: np.ndarray, block_table: np.ndarray, lengths: np.ndarray, page_size: int) -> None:
    """Fill every cache row that no sequence position maps to with bf16 NaN."""
    mapped = np.zeros(kv.shape[0] * page_size, dtype=bool)
    for b in range(block_table.shape[0]):
        L = int(lengths[b])
        if L <= 0:
            continue
        t = np.arange(L)
        phys = block_table[b, t // page_size].astype(np.int64)
        mapped[phys * page_size + t % page_size] = True
    flat = kv.reshape(-1, kv.shape[-1])
    if kv.dtype == np.uint8:                      # fp8 rows: NaN codes and NaN rope
        flat[~mapped, :D_V] = FP8_NAN
        nan_rope = np.full(D_QK - D_V, BF16_NAN, dtype=np.uint16).view(np.uint8)
        flat[~mapped, D_V:640] = nan_rope
    else:
        flat[~mapped] = BF16_NAN


# The five measured workloads.  Index 0 is the small one the oracle finishes in
# well under a second; index 3 is the long-context case (batch 16, 16 heads,
# 64K tokens) that throughput is quoted on.
CONFIGS = {
    "tiny":      dict(batch=1, q_len=1, num_heads=16, page_size=1024, lengths=1024, out_fp32=True),
    "paged":     dict(batch=16, q_len=1, num_heads=16, page_size=64, lengths=4096),
    "two_token": dict(batch=32, q_len=2, num_heads=16, page_size=64, lengths=16384),
    "long":      dict(batch=16, q_len=1, num_heads=16, page_size=64, lengths=65536),
    "ragged":    dict(batch=64, q_len=1, num_heads=128, page_size=64, lengths=None,
                      ragged_range=(1024, 65536)),
}
CONFIG_ORDER = ["tiny", "paged", "two_token", "long", "ragged"]


def make_config(name: str, seed=None, **overrides) -> Problem:
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    if seed is None:
        seed = CONFIG_ORDER.index(name)
    return make_problem(seed=seed, name=name, **cfg)


# ---------------------------------------------------------------------------- the layer around
D_NOPE = 128            # per-head query/key columns that are not rotary (before absorption)
D_ROPE = 64
D_VOUT = 128            # per-head value width after the up-projection


@dataclass
class LayerInputs:
    """Inputs of the steps on either side of the decode (bf16 bit patterns)."""
    q_nope: np.ndarray   # [B, S_q, H, 128]
    q_pe: np.ndarray     # [B, S_q, H, 64]   (before rotary embedding)
    c_kv: np.ndarray     # [B, S_q, 512]     the new tokens' latent rows
    k_pe: np.ndarray     # [B, S_q, 64]      their rope columns, before rotary embedding
    w_uk: np.ndarray     # [H, 512, 128]     key up-projection, row e = latent column e
    w_uv: np.ndarray     # [H, 128, 512]     value up-projection


def make_layer_inputs(batch: int, q_len: int, num_heads: int, *, seed: int = 0) -> LayerInputs:
    """N(0,1) activations; weights N(0, 1/fan_in) so the projected values are O(1).
    Draw order: q_nope, q_pe, c_kv, k_pe, w_uk, w_uv."""
    rng = np.random.default_rng(seed)
    q_nope = _normal_bf16(rng, batch * q_len * num_heads * D_NOPE).reshape(batch, q_len, num_heads, D_NOPE)
    q_pe = _normal_bf16(rng, batch * q_len * num_heads * D_ROPE).reshape(batch, q_len, num_heads, D_ROPE)
    c_kv = _normal_bf16(rng, batch * q_len * D_V).reshape(batch, q_len, D_V)
    k_pe = _normal_bf16(rng, batch * q_len * D_ROPE).reshape(batch, q_len, D_ROPE)
    w_uk = f32_to_bf16_bits(rng.standard_normal((num_heads, D_V, D_NOPE), dtype=np.float32)
                            * np.float32(1.0 / math.sqrt(D_NOPE)))
    w_uv = f32_to_bf16_bits(rng.standard_normal((num_heads, D_VOUT, D_V), dtype=np.float32)
                            * np.float32(1.0 / math.sqrt(D_V)))
    return LayerInputs(q_nope=q_nope, q_pe=q_pe, c_kv=c_kv, k_pe=k_pe, w_uk=w_uk, w_uv=w_uv)
