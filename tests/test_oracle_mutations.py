"""Plant plausible mistakes in the oracle (on the CPU) and require the pins to catch each one.

A pin set that passes a broken oracle pins nothing; this file shows that every
planted mistake below -- a dropped term, a wrong index, a wrong operand, a
wrong log base -- fails at least one pin.
"""
import numpy as np
import pytest

from oracle import mla_oracle as orc
from tests import oracle_pins as pins


def _attend_variant(kind):
    def attend(q_rows, k_rows, v_rows, scale):
        q = np.asarray(q_rows, dtype=np.float64)
        k = np.asarray(k_rows, dtype=np.float64)
        v = np.asarray(v_rows, dtype=np.float64)
        if k.shape[0] == 0:
            return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
        if kind == "no_scale":
            s = q @ k.T
        elif kind == "scale_twice":
            s = scale * scale * (q @ k.T)
        elif kind == "drop_rope":
            s = scale * (q[:, :512] @ k[:, :512].T)
        else:
            s = scale * (q @ k.T)
        m = s.max(axis=1)
        z = np.exp(s - m[:, None]).sum(axis=1)
        lse = m + (np.log2(z) if kind == "log2" else np.log(z))
        if kind == "lse_is_max":
            lse = m
        if kind == "unnormalised":
            p = np.exp(s - m[:, None])
        elif kind == "wrong_axis":
            mc = s.max(axis=0)
            p = np.exp(s - (mc + np.log(np.exp(s - mc[None, :]).sum(axis=0)))[None, :])
        else:
            p = np.exp(s - lse[:, None])
        return p @ v, lse
    return attend


def _gather_no_block_table(kv_cache, block_table_row, length, page_size):
    t = np.arange(int(length))
    return np.asarray(kv_cache)[t // page_size, t % page_size]


def _gather_reversed_row(kv_cache, block_table_row, length, page_size):
    t = np.arange(int(length))
    pages = np.asarray(block_table_row, dtype=np.int64)[t // page_size]
    return np.asarray(kv_cache)[pages, page_size - 1 - t % page_size]


def _decode_sequence_variant(kind):
    def decode_sequence(q_b, kv_cache, block_table_row, length, softmax_scale, page_size, causal=False):
        s_q, h = q_b.shape[0], q_b.shape[1]
        rows = orc.gather_sequence(kv_cache, block_table_row, length, page_size)
        k = orc.widen_bf16(rows)
        if causal:
            out = np.empty((s_q, h, 512))
            lse = np.empty((s_q, h))
            for i in range(s_q):
                if kind == "causal_off_by_one":
                    vis = max(0, int(length) - s_q + i)
                elif kind == "causal_reversed":
                    vis = max(0, int(length) - i)
                elif kind == "causal_ignored":
                    vis = int(length)
                else:
                    vis = max(0, int(length) - s_q + i + 1)
                out[i], lse[i] = orc.attend(orc.widen_bf16(q_b[i]), k[:vis], k[:vis, :512], softmax_scale)
            return out, lse
        if kind == "heads_tokens_swapped":
            q = orc.widen_bf16(q_b).transpose(1, 0, 2).reshape(s_q * h, 576)
        else:
            q = orc.widen_bf16(q_b).reshape(s_q * h, 576)
        v = k[:, 64:] if kind == "v_last_columns" else k[:, :512]
        out, lse = orc.attend(q, k, v, softmax_scale)
        return out.reshape(s_q, h, 512), lse.reshape(s_q, h)
    return decode_sequence


def _combine_variant(kind):
    def combine(partial_out, partial_lse):
        po = np.asarray(partial_out, dtype=np.float64)
        pl = np.asarray(partial_lse, dtype=np.float64)
        M = pl.max(axis=0)
        w = np.exp(M[None, :] - pl) if kind == "sign" else np.exp(pl - M[None, :])
        w = np.where(np.isfinite(w), w, 0.0)
        tot = w.sum(axis=0)
        lse = M + np.log(tot)
        if kind == "unnormalised":
            return np.einsum("sr,srd->rd", w, po), lse
        return np.einsum("sr,srd->rd", w / tot[None, :], po), lse
    return combine


def _e4m3_variant(kind):
    def decode_e4m3(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = np.where(c >> 7, -1.0, 1.0)
        e = (c >> 3) & 15
        m = (c & 7).astype(np.float64)
        bias = 8 if kind == "bias8" else 7
        normal = (1.0 + m / 8.0) * np.exp2((e - bias).astype(np.float64))
        sub = normal if kind == "no_subnormals" else m * 2.0 ** -9
        out = sign * np.where(e == 0, sub, normal)
        if kind == "no_nan":
            return out
        return np.where((c & 0x7F) == 0x7F, np.nan, out)
    return decode_e4m3


def _widen_fp8_variant(kind):
    def widen_fp8_rows(rows):
        r = np.asarray(rows, dtype=np.uint8)
        L = r.shape[0]
        latent = orc.decode_e4m3(r[:, :512])
        sc = np.ascontiguousarray(r[:, 640:656]).view(np.float32).reshape(L, 4).astype(np.float64)
        if kind == "full_scale":
            factor = sc
        else:
            factor = np.exp2(np.floor(np.log2(sc)))
        if kind == "no_scale":
            factor = np.ones_like(factor)
        if kind == "interleaved_groups":
            latent = latent * np.tile(factor, (1, 128))
        else:
            latent = latent * np.repeat(factor, 128, axis=1)
        start = 514 if kind == "rope_offset" else 512
        rope_bytes = np.ascontiguousarray(r[:, start:start + 128])
        rope = orc.widen_bf16(rope_bytes.view(np.uint16).reshape(L, 64))
        return np.concatenate([latent, rope], axis=1)
    return widen_fp8_rows


MUTANTS = {
    "no_scale": ("attend", _attend_variant("no_scale")),
    "scale_twice": ("attend", _attend_variant("scale_twice")),
    "drop_rope": ("attend", _attend_variant("drop_rope")),
    "log2": ("attend", _attend_variant("log2")),
    "lse_is_max": ("attend", _attend_variant("lse_is_max")),
    "unnormalised": ("attend", _attend_variant("unnormalised")),
    "wrong_axis": ("attend", _attend_variant("wrong_axis")),
    "no_block_table": ("gather_sequence", _gather_no_block_table),
    "reversed_row": ("gather_sequence", _gather_reversed_row),
    "v_last_columns": ("decode_sequence", _decode_sequence_variant("v_last_columns")),
    "heads_tokens_swapped": ("decode_sequence", _decode_sequence_variant("heads_tokens_swapped")),
    "causal_off_by_one": ("decode_sequence", _decode_sequence_variant("causal_off_by_one")),
    "causal_reversed": ("decode_sequence", _decode_sequence_variant("causal_reversed")),
    "causal_ignored": ("decode_sequence", _decode_sequence_variant("causal_ignored")),
    "e4m3_bias8": ("decode_e4m3", _e4m3_variant("bias8")),
    "e4m3_no_subnormals": ("decode_e4m3", _e4m3_variant("no_subnormals")),
    "e4m3_no_nan": ("decode_e4m3", _e4m3_variant("no_nan")),
    "fp8_full_scale": ("widen_fp8_rows", _widen_fp8_variant("full_scale")),
    "fp8_no_scale": ("widen_fp8_rows", _widen_fp8_variant("no_scale")),
    "fp8_interleaved_groups": ("widen_fp8_rows", _widen_fp8_variant("interleaved_groups")),
    "fp8_rope_offset": ("widen_fp8_rows", _widen_fp8_variant("rope_offset")),
    "combine_sign": ("combine", _combine_variant("sign")),
    "combine_unnormalised": ("combine", _combine_variant("unnormalised")),
}


def _caught(run):
    try:
        run()
    except (AssertionError, IndexError, ValueError, FloatingPointError):
        return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        if attr == "combine":
            if _caught(lambda: pins.split_combine(orc.attend, orc.combine)):
                caught.append("split_combine")
        else:
            if attr == "decode_e4m3":
                for pin in (pins.fp8_decoder_spec_values, pins.fp8_decoder_matches_torch):
                    if _caught(lambda: pin(orc.decode_e4m3)):
                        caught.append(pin.__name__)
            if attr == "widen_fp8_rows" and _caught(lambda: pins.fp8_scale_exponent_only(orc.widen_fp8_rows)):
                caught.append("fp8_scale_exponent_only")
            for pin in pins.ALL_DECODE_PINS:
                if caught:
                    break
                if _caught(lambda: pin(orc.decode)):
                    caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
