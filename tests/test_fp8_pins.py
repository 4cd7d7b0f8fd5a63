"""Pins of the FP8 (E4M3) part of the oracle (CPU): the decoder of the attention
oracle and the quantiser of the append oracle, checked against the E4M3
conversions of a library (torch ``float8_e4m3fn``) and against what the
format's definition fixes, plus planted mistakes that must fail.

Source of the row: [GITREAD] "TokenSpeed 深度解析:把 LLM 推理压到"光速"意味着什么",
section "核心技术揭秘" (FP8 KV-cache quantisation).  The format reading (OCP
E4M3, finite variant, one fp32 scale per row, scale = max|x| / 448) is the
oracle's."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.kv_append import e4m3_round


def _torch_value(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_round(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def test_decoder_matches_library_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_value(codes)
    got = np.array([oracle.e4m3_value(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decoder_landmarks():
    # the format's fixed points: 0, 1, the smallest subnormal and normal, the largest value
    for code, v in [(0x00, 0.0), (0x38, 1.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0x7E, 448.0),
                    (0xFE, -448.0), (0x07, 7 * 2.0 ** -9), (0x3C, 1.5)]:
        assert oracle.e4m3_value(code) == v, hex(code)


def _check_round(rnd):
    """Raise AssertionError when an E4M3 rounding breaks what the format fixes."""
    vals = _torch_value(FINITE)
    # every representable value is its own code
    assert np.array_equal(rnd(vals.astype(np.float32)), _torch_round(vals.astype(np.float32)))
    # every midpoint between neighbours goes to the even mantissa, as the library rounds
    pos = np.unique(vals[vals >= 0])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[1:] + pos[:-1]) / 2)  # exact in fp32
    for sgn in (1, -1):
        assert np.array_equal(rnd(sgn * mids), _torch_round(sgn * mids))
    # random values over the whole range, subnormals included
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(100000) * np.exp2(rng.uniform(-14, 9, 100000))).astype(np.float32)
    x = x[np.abs(x) < 464]
    assert np.array_equal(rnd(x), _torch_round(x))
    # saturation above the largest value (the library gives NaN past 464)
    assert np.all(rnd(np.array([449.0, 463.9, 500.0, 1e30], np.float32)) == 0x7E)
    assert np.all(rnd(np.array([-449.0, -1e30], np.float32)) == 0xFE)


def test_rounding_pins():
    _check_round(e4m3_round)


def _check_quantizer(q):
    rng = np.random.default_rng(12)
    for std in (1.0, 1e-3, 37.0):
        for _ in range(10):
            x = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal(576).astype(np.float32) * np.float32(std)))
            codes, scale = q(x)
            scale = np.float32(scale)
            i = int(np.argmax(np.abs(x)))
            assert codes[i] == (0x7E if x[i] > 0 else 0xFE)            # the max maps to +-448
            assert np.all((codes & 0x7F) != 0x7F)                      # never NaN
            dec = _torch_value(codes) * np.float64(scale)
            # nearest E4M3 value of the fp32 quotient: half a grid step (relative 2^-4
            # in the normal range, 2^-10 absolute below it) plus the division's rounding
            q64 = x.astype(np.float64) / np.float64(scale)
            step = np.where(np.abs(q64) >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(np.abs(q64), 2.0 ** -6))) - 3),
                            2.0 ** -9)
            assert np.all(np.abs(dec - x) <= (0.5 * step + 448 * 2.0 ** -24) * np.float64(scale) * (1 + 1e-6))
            assert abs(np.float64(scale) * 448 - np.max(np.abs(x))) <= 2 ** -22 * np.max(np.abs(x))
            c2, s2 = q(x * np.float32(8.0))
            assert np.array_equal(c2, codes) and np.float32(s2) == np.float32(8.0) * scale
            c3, s3 = q(-x)
            assert np.array_equal(c3 & 0x7F, codes & 0x7F) and np.float32(s3) == scale
    codes, scale = q(np.zeros(576, np.float32))
    assert np.all((codes & 0x7F) == 0) and np.float32(scale) == np.float32(1.0)


def test_quantizer_pins():
    _check_quantizer(oracle.quantize_row_fp8)


# ---------------- planted mistakes ----------------

def _round_trunc(v):
    v = np.asarray(v, np.float32).astype(np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    grid = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    r = np.minimum(np.floor(a / grid) * grid, 448.0)
    return e4m3_round(np.copysign(r, v).astype(np.float32))


def _round_half_away(v):
    v = np.asarray(v, np.float32).astype(np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    grid = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    r = np.minimum(np.floor(a / grid + 0.5) * grid, 448.0)
    return e4m3_round(np.copysign(r, v).astype(np.float32))


def _round_no_subnormal(v):
    c = e4m3_round(v)
    return np.where((c & 0x78) == 0, c & 0x80, c).astype(np.uint8)


def _round_bias8(v):   # the other common E4M3 variant's exponent bias
    return e4m3_round(np.asarray(v, np.float32) * np.float32(2.0))


@pytest.mark.parametrize("mutant", [_round_trunc, _round_half_away, _round_no_subnormal, _round_bias8])
def test_rounding_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        _check_round(mutant)


def _q_div127(x):
    s = np.float32(np.max(np.abs(x)) / np.float32(127.0)) or np.float32(1.0)
    return e4m3_round(np.asarray(x, np.float32) / s), s


def _q_nosign(x):
    c, s = oracle.quantize_row_fp8(x)
    return (c & 0x7F).astype(np.uint8), s


def _q_trunc(x):
    s = np.float32(np.max(np.abs(x)) / np.float32(448.0)) or np.float32(1.0)
    return _round_trunc(np.asarray(x, np.float32) / s), s


@pytest.mark.parametrize("mutant", [_q_div127, _q_nosign, _q_trunc])
def test_quantizer_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        _check_quantizer(mutant)


# ---------------- the attention oracle on an FP8 cache ----------------

def test_fp8_cache_equals_bf16_cache_of_the_same_values():
    """With scale 1 and codes whose values are exact in bf16 (all of them are),
    attention over the FP8 cache equals attention over the bf16 cache holding
    the decoded values, bit for bit in the oracle."""
    c = synth.make_decode_case(21, batch=2, heads=4, q_len=2, seq_lens=[150, 77], kv_dtype="fp8")
    c.cache.scale[:] = np.float32(1.0)
    ref_out, ref_lse = oracle.decode(c)
    vals = _torch_value(c.cache.data.reshape(-1)).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16).reshape(c.cache.data.shape)
    assert np.array_equal(synth.bf16_to_f32(bits).reshape(-1), vals)  # exact in bf16
    o2, l2 = oracle.attention(c.q, bits, None, c.cache.page_table, c.q_start(), c.cache.kv_lens, c.softmax_scale)
    assert np.array_equal(o2, ref_out) and np.array_equal(l2, ref_lse)


def test_fp8_scale_multiplies_rows():
    """A power-of-two row scale equals the same factor folded into the values."""
    c = synth.make_decode_case(22, batch=1, heads=4, q_len=1, seq_lens=[100], kv_dtype="fp8")
    c.cache.scale[:] = np.float32(0.25)
    out, lse = oracle.decode(c)
    c.cache.scale[:] = np.float32(1.0)
    c.softmax_scale = c.softmax_scale * 0.25
    _, lse2 = oracle.decode(c)
    assert np.allclose(lse, lse2, atol=1e-12)
