"""The oracle of the steps around the decode, against its pins (CPU)."""
import numpy as np
import pytest

from oracle import mla_layer as L
from oracle import mla_oracle as orc
from tests import layer_pins as pins


def test_rope():
    pins.rope_pins(L.rope)


def test_absorption_equals_decompressed_attention():
    pins.absorption_pin(L.q_absorb, L.out_absorb, orc.decode)


def test_fp8_encoding():
    pins.fp8_encoding_pins(L.encode_e4m3, L.fp8_group_exponent)


def test_append():
    pins.append_pins(L.append_rows)


def test_bf16_rounding():
    pins.bf16_rounding_pins(L._f64_to_bf16_bits)


def _rope_variant(kind):
    def rope(x, pos, base=10000.0):
        x = np.asarray(x, dtype=np.float64)
        i = np.arange(32, dtype=np.float64)
        inv = np.power(float(base), -2.0 * i / (64 if kind != "wrong_dim" else 32))
        ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
        c, s = np.cos(ang), np.sin(ang)
        if kind == "halves":
            x0, x1 = x[..., :32], x[..., 32:]
        else:
            x0, x1 = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        a, b = x0 * c - x1 * s, x0 * s + x1 * c
        if kind == "sign":
            a, b = x0 * c + x1 * s, -x0 * s + x1 * c
        if kind == "halves":
            out[..., :32], out[..., 32:] = a, b
        else:
            out[..., 0::2], out[..., 1::2] = a, b
        return out
    return rope


def _q_absorb_transposed(q_nope, q_pe, w_uk, positions, base=10000.0):
    qn = orc.widen_bf16(q_nope)
    w = orc.widen_bf16(w_uk).reshape(w_uk.shape[0], 128, 512)       # a transposed reading of the layout
    lat = np.einsum("bshd,hde->bshe", qn, w)
    pe = L.rope(orc.widen_bf16(q_pe), np.asarray(positions)[:, :, None], base)
    return np.concatenate([lat, pe], axis=-1)


def _out_absorb_other_head(out_latent, w_uv):
    w = orc.widen_bf16(w_uv)[::-1]
    return np.einsum("bshe,hve->bshv", np.asarray(out_latent, dtype=np.float64), w)


def _encode_ties_up(x):
    out = L.encode_e4m3(x)
    vals = orc.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    a = np.abs(np.asarray(x, dtype=np.float64))
    tie = np.isin(a, mids)
    return np.where(tie, (out & 0x7F) + np.where((out & 1) == 0, 1, 0) | (out & 0x80), out).astype(np.uint8)


def _bf16_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    q = np.sign(m) * np.floor(np.abs(m) * 256.0 + 0.5)
    y = (q / 256.0) * np.exp2(e.astype(np.float64))
    return (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_double_rounding(x):
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _bf16_truncating(x):
    return (np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _exponent_off_by_one(amax):
    return L.fp8_group_exponent(amax) + (1 if amax != 0 else 0)


@pytest.mark.parametrize("name", ["rope_sign", "rope_halves", "rope_wrong_dim", "q_absorb_transposed",
                                  "out_absorb_other_head", "encode_ties_up", "exponent_off_by_one",
                                  "bf16_ties_away", "bf16_double_rounding", "bf16_truncating"])
def test_layer_pins_catch_planted_mistake(name, monkeypatch):
    caught = False
    try:
        if name.startswith("rope_"):
            monkeypatch.setattr(L, "rope", _rope_variant(name[5:]))
            pins.rope_pins(L.rope)
        elif name == "q_absorb_transposed":
            pins.absorption_pin(_q_absorb_transposed, L.out_absorb, orc.decode)
        elif name == "out_absorb_other_head":
            pins.absorption_pin(L.q_absorb, _out_absorb_other_head, orc.decode)
        elif name == "encode_ties_up":
            pins.fp8_encoding_pins(_encode_ties_up, L.fp8_group_exponent)
        elif name == "exponent_off_by_one":
            pins.fp8_encoding_pins(L.encode_e4m3, _exponent_off_by_one)
        elif name.startswith("bf16_"):
            pins.bf16_rounding_pins({"bf16_ties_away": _bf16_ties_away, "bf16_double_rounding": _bf16_double_rounding,
                                     "bf16_truncating": _bf16_truncating}[name])
    except AssertionError:
        caught = True
    assert caught, f"planted mistake {name!r} passed the pins"
