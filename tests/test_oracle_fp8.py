"""Pins of the oracle's FP8 (E4M3 x fp32 scale) dequantization and GEMV, each
against something other than the oracle's own formula: torch's E4M3 decode
with the tile looked up element by element, exact rational brute force, closed
forms and invariants."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def torch_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def tiled_case(n, k, seed, tiled=True):
    g = synth.rng(seed)
    w = synth.fp8_weights(g, n, k, tiled=tiled)
    # distinct, non-symmetric tile scales (a transposed or shifted grid changes values)
    w["scales"] = (np.arange(1, w["scales"].size + 1, dtype=np.float32).reshape(w["scales"].shape) * 0.375)
    return w


@pytest.mark.parametrize("n,k,tiled", [(300, 384, True), (130, 160, True), (5, 64, False)])
def test_dequant_matches_torch_decode_and_tile_lookup(n, k, tiled):
    w = tiled_case(n, k, n + k, tiled)
    v = torch_e4m3(w["codes"])
    want = np.empty((n, k))
    for r in range(n):
        for c in range(k):
            s = w["scales"][r // 128, c // 128] if tiled else w["scales"][0, 0]
            want[r, c] = v[r, c] * float(s)
    got = oracle.ops.dequant_fp8(w)
    assert np.array_equal(got, want)


def test_gemv_exact_brute_force_across_tiles():
    n, k, m = 130, 256, 2  # 2 x 2 tiles, the second row of tiles partial
    w = tiled_case(n, k, 5)
    x_bits = synth.x_bf16(synth.rng(6), m, k)
    xv = [[Fraction(float(v)) for v in row] for row in oracle.decode_bf16(x_bits)]
    v = torch_e4m3(w["codes"])
    y = oracle.ops.gemv(w, x_bits)
    for t in range(m):
        for r in range(0, n, 7):
            exact = sum(Fraction(float(v[r, c])) * Fraction(float(w["scales"][r // 128, c // 128])) * xv[t][c]
                        for c in range(k))
            mag = sum(abs(Fraction(float(v[r, c])) * xv[t][c]) for c in range(k)) * 2
            assert abs(Fraction(float(y[t, r])) - exact) <= mag * Fraction(1, 2 ** 45)


@pytest.mark.parametrize("col", [0, 15, 16, 127, 128, 255])
def test_one_hot_column_gives_the_weight(col):
    n, k = 200, 256
    w = tiled_case(n, k, 11)
    x = np.zeros((1, k), np.float32)
    x[0, col] = 1.0
    y = oracle.ops.gemv(w, x)[0]
    want = torch_e4m3(w["codes"][:, col]) * w["scales"][np.arange(n) // 128, col // 128].astype(np.float64)
    assert np.array_equal(y, want)


def test_tensor_scale_equals_uniform_tiles():
    g = synth.rng(3)
    w = synth.fp8_weights(g, 260, 384, tiled=True)
    w["scales"][:] = np.float32(0.0078125)
    wt = dict(w, tiled=False, scales=np.array([[0.0078125]], np.float32))
    x = synth.x_bf16(g, 3, 384)
    assert np.array_equal(oracle.ops.gemv(w, x), oracle.ops.gemv(wt, x))


def test_special_codes():
    w = {"fmt": "fp8", "tiled": False, "codes": np.array([[0x7E, 0xFE, 0x7F, 0x00, 0x80, 0x01] + [0] * 26], np.uint8),
         "scales": np.array([[2.0]], np.float32)}
    d = oracle.ops.dequant_fp8(w)[0]
    assert d[0] == 896.0 and d[1] == -896.0 and np.isnan(d[2])  # max finite 448; 0x7F is NaN
    assert d[3] == 0.0 and d[4] == 0.0 and np.signbit(d[4]) and d[5] == 2.0 ** -8  # -0; smallest subnormal


def test_generator_codes_are_finite_and_in_range():
    w = synth.fp8_weights(synth.rng(9), 300, 384)
    v = torch_e4m3(w["codes"])
    assert np.isfinite(v).all() and np.abs(v).max() <= 448
    # every tile reaches its scale's full range (the max element maps to 448)
    per_tile = np.zeros(w["scales"].shape)
    for i in range(w["scales"].shape[0]):
        for j in range(w["scales"].shape[1]):
            per_tile[i, j] = np.abs(v[128 * i:128 * i + 128, 128 * j:128 * j + 128]).max()
    assert (per_tile == 448).all()
