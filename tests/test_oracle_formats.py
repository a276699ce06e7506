"""Pins of the oracle's format decoders against library decoders, the OCP value
table and exact rational rounding (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import load_golden
from tests.exact import to_bf16, to_f32

pytestmark = pytest.mark.cpu


def test_e2m1_matches_ocp_table():
    table = load_golden("e2m1_values.json")["values"]
    got = oracle.decode_e2m1(np.arange(16))
    assert got.tolist() == table
    # code 8 is negative zero, code 0 positive zero
    assert np.signbit(got[8]) and not np.signbit(got[0])
    # every value times 2 is an integer (the property the integer decode relies on)
    assert np.all(got * 2 == np.round(got * 2))


def test_e4m3_all_256_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    # spot values of the OCP E4M3 definition
    assert got[0x38] == 1.0 and got[0x40] == 2.0 and got[0x7E] == 448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_is_not_the_fnuz_variant():
    # 0x80 is -0 in E4M3 ("FN"); in the FNUZ variant it would be NaN.
    v = oracle.decode_e4m3(np.array([0x80]))
    assert v[0] == 0.0 and np.signbit(v[0])
    fnuz = torch.tensor([0x38], dtype=torch.uint8).view(torch.float8_e4m3fnuz).float().item()
    assert fnuz == 0.5 and oracle.decode_e4m3(np.array([0x38]))[0] == 1.0


def test_fp16_all_65536_against_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.decode_f16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_bf16_all_65536_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_round_to_bf16_matches_torch_on_fp32_inputs():
    g = np.random.default_rng(7)
    v = np.concatenate([
        g.standard_normal(20000),
        g.standard_normal(2000) * 1e-38,   # bf16 subnormal range
        g.standard_normal(2000) * 1e30,
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(v.astype(np.float64))
    assert np.array_equal(ref, got)


@pytest.mark.parametrize("val", [
    Fraction(1) + Fraction(1, 2 ** 8),                         # tie -> even (1.0)
    Fraction(1) + Fraction(3, 2 ** 8),                         # tie -> even (1 + 2^-6)
    Fraction(1) + Fraction(1, 2 ** 8) + Fraction(1, 2 ** 30),  # just above a tie
    -(Fraction(3) + Fraction(1, 2 ** 7)),
    Fraction(5, 2 ** 135),                                     # subnormal
])
def test_round_to_bf16_exact(val):
    got = oracle.round_to_bf16(np.array([float(val)]))[0]
    assert Fraction(got) == to_bf16(val)


def test_round_to_bf16_rounds_once():
    # 1 + 2^-8 + 2^-30 rounds up to 1 + 2^-7 in one step; going through fp32
    # first would land on the tie 1 + 2^-8 and then round to even (1.0).
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.round_to_bf16(np.array([v]))[0] == 1.0 + 2.0 ** -7
    assert Fraction(float(np.float32(v))) == to_f32(Fraction(v))


def test_bf16_ulp():
    assert oracle.bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert oracle.bf16_ulp(np.array([1.99]))[0] == 2.0 ** -7
    assert oracle.bf16_ulp(np.array([2.0]))[0] == 2.0 ** -6
    assert oracle.bf16_ulp(np.array([-0.75]))[0] == 2.0 ** -8
