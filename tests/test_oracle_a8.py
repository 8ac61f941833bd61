"""Pins of the W8A8 activation quantizer and block (page "开源 APXInf 把 VLA 推理
压到 26 毫秒": FP8 applied to weights and activations). Reading: per-token
scale max|x| / 448, round to the nearest E4M3FN value with ties to the even
code, decision in float32. Checked against the format's definition (value
grid, largest magnitude, tie rule), the scale's invariances, an independent
table encoder, and the block's closeness to the unquantized block."""

import dataclasses

import numpy as np
import pytest

from oracle import llm
from oracle.fp8 import decode_e4m3fn, encode_e4m3fn_nearest, fake_quant_act_rows, quantize_act_rows
from oracle.io import Weights, to_f64
from synth import make_inputs, make_weights, small_config
from synth.fp8 import encode_e4m3fn_table


def test_row_maximum_maps_to_448_and_back(rng):
    x = rng.standard_normal((6, 40)) * np.array([1e-3, 1.0, 7.0, 300.0, 2e4, 0.5])[:, None]
    codes, scale = quantize_act_rows(x)
    x32 = x.astype(np.float32)
    for r in range(6):
        j = np.argmax(np.abs(x32[r]))
        assert codes[r, j] in (0x7E, 0xFE)                       # +-448, the largest finite value
        np.testing.assert_allclose(decode_e4m3fn(codes[r, j]) * scale[r], x32[r, j], rtol=2e-7)
        assert scale[r] == np.float32(np.abs(x32[r]).max() / np.float32(448.0))


def test_values_are_on_the_grid_within_half_a_step(rng):
    x = rng.standard_normal((4, 512)) * 3.0
    codes, scale = quantize_act_rows(x)
    y = x.astype(np.float32) * (np.float32(448.0) / np.abs(x.astype(np.float32)).max(axis=1))[:, None]
    v = decode_e4m3fn(codes)
    assert np.isfinite(v).all() and np.abs(v).max() <= 448.0
    # grid step at |y|: 2^(e-3) in binade [2^e, 2^(e+1)), 2^-9 below 2^-6
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
    step = np.where(np.abs(y) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))
    assert (np.abs(v - y) <= step / 2 * (1 + 1e-12)).all()


def test_ties_go_to_the_even_code():
    # midpoints between neighbouring grid values: 1 + 1/16 lies between 1 (0x38)
    # and 1.125 (0x39); 1.1875 between 1.125 (0x39) and 1.25 (0x3A); 2^-9 / 2
    # between 0 and the smallest subnormal
    assert encode_e4m3fn_nearest(np.array([1.0625]))[0] == 0x38
    assert encode_e4m3fn_nearest(np.array([1.1875]))[0] == 0x3A
    assert encode_e4m3fn_nearest(np.array([2.0 ** -10]))[0] == 0x00
    assert encode_e4m3fn_nearest(np.array([-1.0625]))[0] == 0xB8
    assert encode_e4m3fn_nearest(np.array([464.0, -1e9]))[:].tolist() == [0x7E, 0xFE]   # saturation


def test_matches_an_independent_table_encoder(rng):
    y = np.concatenate([rng.standard_normal(4000) * 50, rng.uniform(-1e-2, 1e-2, 1000),
                        np.array([0.0, -0.0, 448.0, -448.0, 500.0])])
    got = encode_e4m3fn_nearest(y)
    # same magnitude codes; the sign bit is the value's (negative values that
    # round to zero are -0 here, +0 in the weight-storage encoder)
    assert np.array_equal(got & 0x7F, encode_e4m3fn_table(y) & 0x7F)
    assert np.array_equal((got & 0x80) != 0, np.signbit(y))


def test_zero_rows_and_power_of_two_scaling(rng):
    x = rng.standard_normal((3, 64))
    x[1] = 0.0
    codes, scale = quantize_act_rows(x)
    assert (codes[1] == 0).all() and scale[1] == 0.0 and (fake_quant_act_rows(x)[1] == 0).all()
    c2, s2 = quantize_act_rows(x * 2.0 ** 7)
    assert np.array_equal(c2, codes)
    assert np.array_equal(s2, scale * np.float32(2.0 ** 7))


def test_rows_are_quantized_independently(rng):
    x = rng.standard_normal((5, 96))
    y = x.copy()
    y[2] *= 1e3                                   # one token far larger than the rest
    a, b = fake_quant_act_rows(x), fake_quant_act_rows(y)
    keep = [0, 1, 3, 4]
    assert np.array_equal(a[keep], b[keep])


def test_a8_block_is_close_to_the_unquantized_block(rng):
    cfg = small_config("block", "fp8", seq=37)
    W = Weights(make_weights(cfg))
    x = to_f64(make_inputs(cfg)["x"])
    plain = llm.block(x, W, "llm.0.", cfg.block)
    a8 = llm.block(x, W, "llm.0.", dataclasses.replace(cfg.block, a8="fp8"))
    d = np.linalg.norm(a8 - plain) / np.linalg.norm(plain - x)     # relative to the block's update
    # four quantized inputs of about 2^-5 relative rounding each: a few percent, not zero
    assert 1e-3 < d < 0.1, d
