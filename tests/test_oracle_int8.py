"""Pins of the INT8 variant (page "开源 APXInf 把 VLA 推理压到 26 毫秒": INT8 where
FP8 units are missing). Weights: int8 codes with a per-channel scale
max|row| / 127. Activations: per-token scale max|x| / 127, nearest integer
(halves to even) decided in float32, clipped to 127. Checked against the
integer grid's definition (row maximum, half-step bound, tie rule), the
scale's invariances, per-row independence and closeness of the int8 block to
the unquantized one."""

import dataclasses

import numpy as np

from oracle import llm
from oracle.int8 import fake_quant_act_rows, quantize_act_rows
from oracle.io import Weights, to_f64
from synth import make_inputs, make_weights, small_config
from synth.int8 import quantize_rows


def test_weight_storage_round_trip(rng):
    w = rng.standard_normal((20, 96)).astype(np.float32) * np.logspace(-3, 2, 20, dtype=np.float32)[:, None]
    codes, scale = quantize_rows(w)
    assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() == 127
    back = codes.astype(np.float64) * scale.astype(np.float64)[:, None]
    assert (np.abs(back - w) <= scale[:, None].astype(np.float64) / 2 * (1 + 1e-6)).all()


def test_row_maximum_maps_to_127_and_values_within_half_a_step(rng):
    x = rng.standard_normal((6, 200)) * np.array([1e-3, 1.0, 7.0, 300.0, 2e4, 0.5])[:, None]
    codes, scale = quantize_act_rows(x)
    x32 = x.astype(np.float32)
    for r in range(6):
        j = np.argmax(np.abs(x32[r]))
        assert abs(int(codes[r, j])) == 127
        assert scale[r] == np.float32(np.abs(x32[r]).max() / np.float32(127.0))
    y = x32 * (np.float32(127.0) / np.abs(x32).max(axis=1))[:, None]
    assert (np.abs(codes - y) <= 0.5 * (1 + 1e-6)).all()


def test_ties_go_to_even():
    x = np.array([[127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 126.5]], dtype=np.float32)   # multiplier exactly 1
    codes, _ = quantize_act_rows(x)
    assert codes[0].tolist() == [127, 2, 4, -2, -4, 0, 0, 126]


def test_zero_rows_power_of_two_scaling_and_row_independence(rng):
    x = rng.standard_normal((4, 64))
    x[1] = 0.0
    codes, scale = quantize_act_rows(x)
    assert (codes[1] == 0).all() and scale[1] == 0.0
    c2, s2 = quantize_act_rows(x * 2.0 ** -5)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scale * np.float32(2.0 ** -5))
    y = x.copy()
    y[2] *= 1e3
    keep = [0, 1, 3]
    assert np.array_equal(fake_quant_act_rows(x)[keep], fake_quant_act_rows(y)[keep])


def test_int8_block_is_close_to_the_unquantized_block():
    cfg = small_config("block", "int8", seq=37)
    W = Weights(make_weights(cfg))
    x = to_f64(make_inputs(cfg)["x"])
    plain = llm.block(x, W, "llm.0.", cfg.block)
    q = llm.block(x, W, "llm.0.", dataclasses.replace(cfg.block, a8="int8"))
    d = np.linalg.norm(q - plain) / np.linalg.norm(plain - x)
    # four quantized inputs at 7 bits: about a percent, not zero
    assert 1e-4 < d < 0.05, d
