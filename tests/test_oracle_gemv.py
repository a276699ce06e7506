"""Pins of the oracle's dequantization and GEMV (CPU only): hand-worked examples,
exact rational brute force on tiny shapes, and closed-form special cases."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import load_golden

pytestmark = pytest.mark.cpu

E2M1 = [Fraction(v).limit_denominator() for v in load_golden("e2m1_values.json")["values"]]


def _ex(id_):
    for e in load_golden("worked_examples.json")["examples"]:
        if e["id"] == id_:
            return e
    raise KeyError(id_)


def _bf16(vals):
    return synth.to_bf16_bits(np.asarray(vals, dtype=np.float32))


# ---------------------------------------------------------------- worked examples

def test_ex1_nvfp4_one_block():
    for id_ in ("EX-1a", "EX-1b"):
        e = _ex(id_)
        w = {"fmt": "nvfp4", "codes": np.array(e["codes"], np.uint8),
             "scales": np.array(e["scales"], np.uint8), "tensor_scale": np.float32(e["tensor_scale"])}
        y = oracle.gemv(w, _bf16(e["x"]))
        assert y.tolist() == e["y"], id_


def test_ex2_q8_0_one_block():
    j = np.arange(32)
    for id_, x in (("EX-2a", j.astype(np.float32)), ("EX-2b", np.ones(32, np.float32))):
        e = _ex(id_)
        w = {"fmt": "q8_0", "codes": (j - 16).astype(np.int8)[None], "scales": np.array(e["scales"], np.uint16)}
        assert oracle.gemv(w, x[None]).tolist() == e["y"], id_


def test_ex3_q4_0_one_block():
    e = _ex("EX-3")
    w = {"fmt": "q4_0", "codes": (np.arange(32) % 16).astype(np.uint8)[None],
         "scales": np.array(e["scales"], np.uint16)}
    assert oracle.gemv(w, np.ones((1, 32), np.float32)).tolist() == e["y"]


def test_ex6_nvfp4_two_rows_two_blocks_pins_scale_indexing():
    e = _ex("EX-6")
    w = {"fmt": "nvfp4", "codes": np.array(e["codes"], np.uint8),
         "scales": np.array(e["scales"], np.uint8), "tensor_scale": np.float32(e["tensor_scale"])}
    x = _bf16([[1.0] * 16 + [2.0] * 16])
    assert oracle.gemv(w, x).tolist() == e["y"]


def test_ex7_q8_0_two_rows_two_blocks():
    e = _ex("EX-7")
    codes = np.zeros((2, 64), np.int8)
    codes[0, :32], codes[0, 32:], codes[1, :32], codes[1, 32:] = 1, -2, 3, 5
    w = {"fmt": "q8_0", "codes": codes, "scales": np.array(e["scales"], np.uint16)}
    x = np.array([[1.0] * 32 + [-1.0] * 32], np.float32)
    assert oracle.gemv(w, x).tolist() == e["y"]


def test_ex8_q4_0_two_rows_two_blocks():
    e = _ex("EX-8")
    codes = np.zeros((2, 64), np.uint8)
    codes[0, :32], codes[0, 32:], codes[1, :32], codes[1, 32:] = 9, 0, 15, 8
    w = {"fmt": "q4_0", "codes": codes, "scales": np.array(e["scales"], np.uint16)}
    x = np.array([[1.0] * 32 + [2.0] * 32], np.float32)
    assert oracle.gemv(w, x).tolist() == e["y"]


# ---------------------------------------------------------------- exact brute force

def _e4m3_fraction(b):
    s, e, m = (b >> 7) & 1, (b >> 3) & 15, b & 7
    mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


def _f16_fraction(u):
    s, e, m = (u >> 15) & 1, (u >> 10) & 31, u & 1023
    mag = Fraction(m, 1024) * Fraction(1, 2 ** 14) if e == 0 else (1 + Fraction(m, 1024)) * Fraction(2) ** (e - 15)
    return -mag if s else mag


def _x_fractions(x):
    """Activation values as rationals, decoded by library casts (not the oracle)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        import torch
        v = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    else:
        v = x.astype(np.float64)
    return [[Fraction(float(t)) for t in row] for row in v]


def _brute_nvfp4(w, x):
    """Element-by-element exact sum: every weight decoded on its own with rationals."""
    n, k = w["codes"].shape
    st = Fraction(float(np.float32(w["tensor_scale"])))
    X = _x_fractions(x)
    out = []
    for xm in X:
        row = []
        for i in range(n):
            acc = Fraction(0)
            for j in range(k):
                wv = E2M1[int(w["codes"][i, j])] * _e4m3_fraction(int(w["scales"][i][j // 16])) * st
                acc += wv * xm[j]
            row.append(acc)
        out.append(row)
    return out


def _brute_q(w, x, offset):
    n, k = w["codes"].shape
    X = _x_fractions(x)
    out = []
    for xm in X:
        row = []
        for i in range(n):
            acc = Fraction(0)
            for j in range(k):
                wv = _f16_fraction(int(w["scales"][i][j // 32])) * (int(w["codes"][i, j]) - offset)
                acc += wv * xm[j]
            row.append(acc)
        out.append(row)
    return out


@pytest.mark.parametrize("n,k,m", [(1, 16, 1), (2, 32, 1), (3, 48, 2), (5, 80, 3), (17, 32, 1)])
def test_nvfp4_gemv_vs_exact(n, k, m):
    g = synth.rng(1000 + n * 7 + k + m)
    w = synth.nvfp4_weights(g, n, k, tensor_scale=0.01)
    x = synth.x_bf16(g, m, k)
    ref = _brute_nvfp4(w, x)
    y = oracle.gemv(w, x)
    for a in range(m):
        for b in range(n):
            # fp64 sum of at most 80 exactly-representable terms
            assert abs(Fraction(float(y[a, b])) - ref[a][b]) <= abs(ref[a][b]) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)


@pytest.mark.parametrize("fmt,n,k,m", [("q8_0", 1, 32, 1), ("q8_0", 3, 64, 2), ("q8_0", 5, 96, 1),
                                       ("q4_0", 1, 32, 1), ("q4_0", 2, 64, 3), ("q4_0", 17, 32, 1)])
def test_q_gemv_vs_exact(fmt, n, k, m):
    g = synth.rng(2000 + n * 7 + k + m)
    w = (synth.q8_0_weights if fmt == "q8_0" else synth.q4_0_weights)(g, n, k)
    x = synth.x_f32(g, m, k)
    ref = _brute_q(w, x, 0 if fmt == "q8_0" else 8)
    y = oracle.gemv(w, x)
    for a in range(m):
        for b in range(n):
            assert abs(Fraction(float(y[a, b])) - ref[a][b]) <= abs(ref[a][b]) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 90)


# ---------------------------------------------------------------- closed forms

def test_one_hot_x_returns_the_weight_column():
    g = synth.rng(5)
    for w in (synth.nvfp4_weights(g, 7, 64), synth.q8_0_weights(g, 7, 64), synth.q4_0_weights(g, 7, 64)):
        D = oracle.ops.dequant(w)
        for col in (0, 17, 63):
            x = np.zeros((1, 64), np.float32)
            x[0, col] = 1.0
            assert np.array_equal(oracle.gemv(w, x)[0], D[:, col])


def test_nvfp4_dequant_f32_is_one_rounding_of_an_exact_product():
    g = synth.rng(6)
    w = synth.nvfp4_weights(g, 4, 64, tensor_scale=0.01)
    f32 = oracle.dequant_nvfp4_f32(w)
    st = Fraction(float(np.float32(0.01)))
    for i in range(4):
        for j in range(64):
            exact = E2M1[int(w["codes"][i, j])] * _e4m3_fraction(int(w["scales"][i, j // 16])) * st
            from tests.exact import to_f32
            assert Fraction(float(f32[i, j])) == to_f32(exact)


def test_zero_inputs_give_zero():
    g = synth.rng(8)
    w = synth.nvfp4_weights(g, 3, 32)
    assert np.all(oracle.gemv(w, np.zeros((2, 32), np.float32)) == 0)
    w["scales"][:] = 0
    assert np.all(oracle.gemv(w, synth.x_bf16(g, 2, 32)) == 0)


def test_power_of_two_scaling_is_exact():
    g = synth.rng(9)
    w = synth.q8_0_weights(g, 4, 64)
    x = synth.x_f32(g, 2, 64)
    assert np.array_equal(oracle.gemv(w, x * np.float32(8.0)), 8.0 * oracle.gemv(w, x))


def test_tolerance_formula():
    assert oracle.tolerance(np.array([0.0]))[0] == 1e-6
    assert oracle.tolerance(np.array([10.0]))[0] == pytest.approx(1e-4 + 1e-6)


def test_nonsquare_orientation():
    # y = W x with W [n, k]: y has n entries per token, and column k of W meets x[k]
    w = {"fmt": "q8_0", "codes": np.zeros((3, 64), np.int8), "scales": np.full((3, 2), 0x3C00, np.uint16)}
    w["codes"][2, 40] = 5
    x = np.zeros((1, 64), np.float32)
    x[0, 40] = 2.0
    assert oracle.gemv(w, x).tolist() == [[0.0, 0.0, 10.0]]
