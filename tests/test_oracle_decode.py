"""Pins for the oracle's storage decoders (bfloat16, FP8 E4M3FN, float32)."""

import math

import numpy as np
import torch

import oracle


def test_bf16_decode_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_decode_spec_points():
    # binary32 with the low half zero: 0x3F80 = 1.0, 0xC000 = -2.0, 0x0001 = 2^-133
    v = oracle.decode_bf16(np.array([0x3F80, 0xC000, 0x0001, 0x7F80], dtype=np.uint16))
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0 ** -133 and math.isinf(v[3])


def test_e4m3fn_spec_points():
    # OCP 8-bit floating point specification, E4M3 (bias 7, no infinities, S.1111.111 = NaN)
    pts = {
        0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
        0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0x77: 240.0, 0x30: 0.5,
    }
    codes = np.array(list(pts.keys()), dtype=np.uint8)
    got = oracle.decode_e4m3fn(codes)
    for c, g in zip(codes, got):
        assert g == pts[int(c)], hex(int(c))
    assert math.copysign(1.0, oracle.decode_e4m3fn(np.array([0x80], np.uint8))[0]) == -1.0
    assert np.isnan(oracle.decode_e4m3fn(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3fn_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_values_are_monotone_in_magnitude():
    pos = oracle.decode_e4m3fn(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert pos[-1] == 448.0


def test_f32_decode_is_exact_widening():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.decode_f32(x), x.astype(np.float64))
