"""Pins of the oracle's activation quantizer and W4A8 integer block dot (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import load_golden
from tests.exact import round_half_even_int, to_f16, to_f32

pytestmark = pytest.mark.cpu


def _ex(id_):
    return next(e for e in load_golden("worked_examples.json")["examples"] if e["id"] == id_)


def test_ex4_quantizer_and_a8_dot():
    e = _ex("EX-4")
    x = np.ones((1, 32), np.float32)
    xq, xd, xs = oracle.quantize_q8_0_act(x)
    assert np.all(xq == 127)
    assert int(xd[0, 0]) == e["xd_bits"]
    assert int(xs[0, 0]) == e["xs"]
    w = {"fmt": "q4_0", "codes": (np.arange(32) % 16).astype(np.uint8)[None],
         "scales": np.array(e["scales"], np.uint16)}
    assert int(oracle.block_isums_q4_0_a8(w, xq)[0, 0, 0]) == e["isum"]
    assert oracle.gemv_q4_0_a8(w, xq, xd).tolist() == e["y"]


def _quantize_exact(block):
    """Q8_0 quantization of one 32-block with every rounding done on rationals."""
    vals = [Fraction(float(v)) for v in block]
    amax = max(abs(v) for v in vals)
    d32 = to_f32(amax / 127)
    d16 = to_f16(d32)
    if d32 == 0:
        return [0] * 32, d16
    q = [max(-127, min(127, round_half_even_int(to_f32(v / d32)))) for v in vals]
    return q, d16


@pytest.mark.parametrize("scale", [1.0, 1e-3, 37.0, 1e-30])
def test_quantizer_vs_exact_rationals(scale):
    g = synth.rng(300 + int(np.log10(scale) + 40))
    x = (synth.x_f32(g, 3, 128) * np.float32(scale)).astype(np.float32)
    x[1, 32:64] = 0.0                 # an all-zero block
    x[2, 5] = x[2, 6] = -np.abs(x[2]).max() * np.float32(1.5)  # repeated amax
    xq, xd, xs = oracle.quantize_q8_0_act(x)
    for m in range(3):
        for b in range(4):
            q, d16 = _quantize_exact(x[m, 32 * b:32 * b + 32])
            assert xq[m, 32 * b:32 * b + 32].tolist() == q
            got_d = Fraction(float(np.uint16(xd[m, b]).view(np.float16)))
            assert got_d == d16
            assert int(xs[m, b]) == sum(q)


def test_quantizer_ties_round_half_even():
    # amax = 127 gives d32 = 1 exactly, so x/d32 = x and the ties are visible
    x = np.zeros((1, 32), np.float32)
    x[0, :6] = [127.0, 0.5, 1.5, 2.5, -0.5, -2.5]
    xq, xd, _ = oracle.quantize_q8_0_act(x)
    assert xq[0, :6].tolist() == [127, 0, 2, 2, 0, -2]
    assert int(xd[0, 0]) == 0x3C00


def test_integer_activations_are_kept_exactly():
    # integer x in [-127, 127] with one +-127 per block: d = 1 and q = x
    g = synth.rng(31)
    x = g.integers(-126, 127, size=(2, 96)).astype(np.float32)
    x[:, ::32] = 127.0
    x[1, 32] = -127.0
    xq, xd, xs = oracle.quantize_q8_0_act(x)
    assert np.array_equal(xq.astype(np.float32), x)
    assert np.all(xd == 0x3C00)
    assert np.array_equal(xs, x.reshape(2, 3, 32).sum(axis=2).astype(np.int32))


def test_block_isums_vs_python_ints():
    g = synth.rng(32)
    w = synth.q4_0_weights(g, 5, 96)
    xq, _, _ = oracle.quantize_q8_0_act(synth.x_f32(g, 3, 96))
    isum = oracle.block_isums_q4_0_a8(w, xq)
    for m in range(3):
        for n in range(5):
            for b in range(3):
                ref = sum((int(w["codes"][n, j]) - 8) * int(xq[m, j]) for j in range(32 * b, 32 * b + 32))
                assert int(isum[m, n, b]) == ref


def test_a8_dot_equals_float_gemv_on_dequantized_activation():
    # identity: sum_b dw*dx*isum_b == sum_k w_k * (dx * q_k)
    g = synth.rng(33)
    w = synth.q4_0_weights(g, 6, 160)
    xq, xd, _ = oracle.quantize_q8_0_act(synth.x_f32(g, 4, 160))
    xhat = (xq.reshape(4, 5, 32) * oracle.decode_f16(xd)[:, :, None]).reshape(4, 160)
    ref = oracle.gemv(w, xhat)
    got = oracle.gemv_q4_0_a8(w, xq, xd)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-15)
    absr = oracle.gemv_abs(w, xhat)
    assert np.allclose(oracle.gemv_q4_0_a8_abs(w, xq, xd), absr, rtol=1e-13, atol=1e-15)


def test_a8_exact_small_integer_case():
    # unit weight scales and integer activations: y is an exact integer
    g = synth.rng(34)
    w = synth.q4_0_weights(g, 3, 64)
    w["scales"][:] = 0x3C00
    x = g.integers(-127, 128, size=(1, 64)).astype(np.float32)
    x[0, 0] = x[0, 32] = 127.0
    xq, xd, _ = oracle.quantize_q8_0_act(x)
    y = oracle.gemv_q4_0_a8(w, xq, xd)
    ref = [[sum((int(w["codes"][n, j]) - 8) * int(x[0, j]) for j in range(64)) for n in range(3)]]
    assert y.tolist() == ref
