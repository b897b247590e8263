"""Pins of the FP8 E4M3 codec (oracle/fp8.py) against the format's
definition: code points of the OCP E4M3 table, the value range, round to
nearest with ties to even, the clamp, NaN kept as the NaN code, dequantised
values worked by hand (per tensor and per KV head), torch's own
float8_e4m3fn conversion on in-range values, and the exactness of
dequantised values in bf16."""
import numpy as np
import pytest
import torch

from oracle import fp8


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x08, 2.0 ** -6), (0x07, 0.875 * 2.0 ** -6), (0x01, 2.0 ** -9),
    (0x40, 2.0), (0x3C, 1.5), (0x77, 240.0), (0x30, 0.5),
])
def test_code_points(code, value):
    assert fp8.decode(code) == value


def test_nan_codes_and_finite_range():
    assert np.isnan(fp8.decode(0x7F)) and np.isnan(fp8.decode(0xFF))
    vals = [fp8.decode(c) for c in range(256) if c not in (0x7F, 0xFF)]
    assert max(vals) == 448.0 and min(vals) == -448.0
    pos = sorted(fp8.decode(c) for c in range(0x00, 0x7F))
    assert pos == sorted(set(pos)) and len(pos) == 127   # all distinct


def test_every_finite_code_round_trips():
    for c in range(256):
        v = fp8.decode(c)
        if np.isnan(v):
            continue
        assert fp8.encode_value(v) == c


@pytest.mark.parametrize("x,code", [
    (1.0 + 1 / 16, 0x38),      # halfway 1.0 / 1.125 -> even mantissa (1.0)
    (1.0 + 3 / 16, 0x3A),      # halfway 1.125 / 1.25 -> even (1.25)
    (2.0 ** -10, 0x00),        # halfway 0 / 2^-9 -> even (0)
    (3 * 2.0 ** -10, 0x02),    # halfway 2^-9 / 2^-8 -> even (2^-8)
    (1.05, 0x38), (1.07, 0x39), (1.1, 0x39), (-1.1, 0xB9),
    (-2.0 ** -11, 0x80),       # rounds to -0
])
def test_round_to_nearest_even(x, code):
    assert fp8.encode_value(x) == code


def test_quantize_clamps_in_fp32():
    x = np.array([1e6, -1e6, 449.0, 448.0, 300.0, np.nan], dtype=np.float32)
    got = fp8.quantize(x, 1.0).tolist()
    assert got[:5] == [0x7E, 0xFE, 0x7E, 0x7E, fp8.encode_value(288.0)]
    assert got[5] == 0x7F                      # NaN stays NaN
    # the product is taken in fp32 before rounding
    x = np.array([3.0], dtype=np.float32)
    inv = np.float32(1 / 3.0)
    assert fp8.quantize(x, inv)[0] == fp8.encode_value(
        float(np.float32(3.0) * inv))


def test_dequantised_values_are_exact_in_bf16():
    vals = np.array([fp8.decode(c) for c in range(256)
                     if not np.isnan(fp8.decode(c))], dtype=np.float32)
    t = torch.from_numpy(vals)
    assert torch.equal(t.to(torch.bfloat16).float(), t)


def test_nan_keeps_its_sign_and_infinities_saturate():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf], dtype=np.float32)
    assert fp8.quantize(x, 0.25).tolist() == [0x7F, 0xFF, 0x7E, 0xFE]


@pytest.mark.parametrize("code,scale,value", [
    (0x38, 0.5, 0.5),                 # 1.0 * 0.5
    (0x7E, 0.01, 4.48),               # 448 * 0.01
    (0xB8, 2.0, -2.0),                # -1.0 * 2
    (0x01, 4.0, 2.0 ** -7),           # 2^-9 * 4
    (0x3C, 3.0, 4.5),                 # 1.5 * 3
    (0xC4, 0.125, -0.375),            # -(1 + 4/8) * 2 * 0.125
    (0x00, 7.0, 0.0),
])
def test_dequantize_by_hand(code, scale, value):
    got = fp8.dequantize(np.array([code]), scale)[0]
    assert got == pytest.approx(value, rel=1e-15, abs=0)


def test_dequantize_nan_code_is_nan():
    assert np.isnan(fp8.dequantize(np.array([0x7F, 0xFF]), 2.0)).all()


def test_per_head_scales_by_hand():
    # rows [T=1, Hkv=2, D=2]; head 0 scale 2 (inv 0.5), head 1 scale 0.25
    # (inv 4): head 0 stores 1.0 * 0.5 = 0.5 (0x30) and 3.0 * 0.5 = 1.5
    # (0x3C); head 1 stores 1.0 * 4 = 4 (0x48) and -0.5 * 4 = -2 (0xC0)
    x = np.array([[[1.0, 3.0], [1.0, -0.5]]], dtype=np.float32)
    inv = np.array([[0.5], [4.0]], dtype=np.float32)
    codes = fp8.quantize(x, inv)
    assert codes.tolist() == [[[0x30, 0x3C], [0x48, 0xC0]]]
    back = fp8.dequantize(codes, np.array([[2.0], [0.25]]))
    assert back.tolist() == [[[1.0, 3.0], [1.0, -0.5]]]


def test_matches_torch_float8_e4m3fn_in_range():
    # torch's conversion (round to nearest even) on fp32 products within the
    # finite range, and on NaN; above 448 torch does not saturate, so those
    # are left out (the saturation is this codec's stated reading)
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 40,
        rng.standard_normal(20000).astype(np.float32) * 0.02,
        np.array([np.nan, -np.nan, 0.0, -0.0, 448.0, -448.0],
                 dtype=np.float32)])
    inv = np.float32(1.0 / 1.7)
    prod = x * inv
    keep = np.isnan(prod) | (np.abs(prod) <= 448.0)
    x, prod = x[keep], prod[keep]
    ref = torch.from_numpy(prod).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    assert np.array_equal(fp8.quantize(x, inv), ref)
