"""Pins of the oracle's K-quant (Q4_K, Q5_K, Q6_K) and IQ4_XS definitions and
of its Q8_0-activation GEMV, each against something other than the oracle's
own vectorised formula: exact rational brute force element by element (with
an independent binary16 decoder), reductions to the Q4_0 / Q8_0 definitions
(pinned on their own elsewhere), one-hot sub-block and super-block cases, and
the integer-dot form of the W4A8 oracle.

The pages name these formats but print no definition, value or example; the
definitions are the public GGUF ones (listed in the design notes).  The
IQ4_XS codebook below is typed from that public definition: it pins the
oracle's indexing and scale offset, not the values themselves (parity
unpinned for the codebook)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.cpu

# The IQ4_NL codebook that IQ4_XS indexes (public GGUF definition).
CODEBOOK = [-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113]


def f16_fraction(bits: int) -> Fraction:
    """IEEE binary16 bits -> exact rational (independent of numpy)."""
    bits = int(bits)
    sign = -1 if bits >> 15 else 1
    e = (bits >> 10) & 31
    f = bits & 1023
    assert e != 31, "no inf/nan scales in these tests"
    if e == 0:
        return sign * Fraction(f, 1 << 24)
    return sign * Fraction(1024 + f, 1 << 10) * (Fraction(2) ** (e - 15))


def brute_value(w: dict, r: int, c: int) -> Fraction:
    """One weight straight from the format definition, in exact arithmetic."""
    fmt = w["fmt"]
    q = int(w["codes"][r, c])
    d = f16_fraction(w["d"][r, c // 256])
    if fmt in (synth.Q4_K, synth.Q5_K):
        dmin = f16_fraction(w["dmin"][r, c // 256])
        return d * int(w["sub"][r, c // 32]) * q - dmin * int(w["mins"][r, c // 32])
    if fmt == synth.Q6_K:
        return d * int(np.int8(w["sub"][r, c // 16])) * (q - 32)
    return d * (int(w["sub"][r, c // 32]) - 32) * CODEBOOK[q]


@pytest.mark.parametrize("fmt", synth.KQUANTS)
def test_dequant_exact_brute_force(fmt):
    w = synth.kquant_weights(synth.rng(11), fmt, 3, 512)
    got = oracle.ops.dequant(w)
    for r in range(3):
        for c in range(512):
            assert Fraction(got[r, c]) == brute_value(w, r, c), (fmt, r, c)


@pytest.mark.parametrize("fmt", synth.KQUANTS)
def test_gemv_a8_exact_brute_force(fmt):
    w = synth.kquant_weights(synth.rng(12), fmt, 2, 256)
    xq, xd, _ = oracle.quantize_q8_0_act(synth.x_f32(synth.rng(13), 2, 256))
    got = oracle.gemv_a8(w, xq, xd)
    for t in range(2):
        for r in range(2):
            exact = sum(brute_value(w, r, c) * f16_fraction(xd[t, c // 32]) * int(xq[t, c]) for c in range(256))
            assert abs(Fraction(got[t, r]) - exact) <= abs(exact) * Fraction(1, 1 << 40) + Fraction(1, 1 << 60)


def test_q4_k_reduces_to_q4_0():
    """sc = 1, m = 8, dmin = d gives d * (q - 8): the Q4_0 rule with d per 32."""
    g = synth.rng(14)
    w = synth.kquant_weights(g, synth.Q4_K, 4, 512)
    w["sub"][:] = 1
    w["mins"][:] = 8
    w["dmin"] = w["d"].copy()
    q40 = {"fmt": "q4_0", "codes": w["codes"], "scales": np.repeat(w["d"], 8, axis=1)}
    assert np.array_equal(oracle.ops.dequant(w), oracle.dequant_q4_0(q40))


def test_q5_k_uses_the_fifth_bit():
    """Q5_K codes 0..31 with sc = 1, m = 16, dmin = d give d * (q - 16): Q8_0 with those codes."""
    g = synth.rng(15)
    w = synth.kquant_weights(g, synth.Q5_K, 4, 512)
    assert (w["codes"] >= 16).any()
    w["sub"][:] = 1
    w["mins"][:] = 16
    w["dmin"] = w["d"].copy()
    q8 = {"fmt": "q8_0", "codes": (w["codes"].astype(np.int16) - 16).astype(np.int8),
          "scales": np.repeat(w["d"], 8, axis=1)}
    assert np.array_equal(oracle.ops.dequant(w), oracle.dequant_q8_0(q8))


def test_q6_k_reduces_to_q8_0():
    """Q6_K with every sub-block scale 1 is d * (q - 32): Q8_0 with codes q - 32."""
    g = synth.rng(16)
    w = synth.kquant_weights(g, synth.Q6_K, 4, 512)
    w["sub"][:] = 1
    q8 = {"fmt": "q8_0", "codes": (w["codes"].astype(np.int16) - 32).astype(np.int8),
          "scales": np.repeat(w["d"], 8, axis=1)}
    assert np.array_equal(oracle.ops.dequant(w), oracle.dequant_q8_0(q8))


@pytest.mark.parametrize("fmt", synth.KQUANTS)
def test_one_hot_sub_block(fmt):
    """Only sub-block j carries a nonzero scale: the weights vanish outside its
    columns and equal the one-scale closed form inside (pins the sub-block
    length and index)."""
    width = 16 if fmt == synth.Q6_K else 32
    k = 512
    for j in (0, 5, k // width - 1):
        w = synth.kquant_weights(synth.rng(17 + j), fmt, 2, k)
        zero = 32 if fmt == synth.IQ4_XS else 0
        w["sub"][:] = zero
        w["sub"][:, j] = zero + 3
        if fmt in (synth.Q4_K, synth.Q5_K):
            w["mins"][:] = 0
        got = oracle.ops.dequant(w)
        cols = np.arange(k)
        inside = (cols >= width * j) & (cols < width * (j + 1))
        assert (got[:, ~inside] == 0).all()
        d = oracle.decode_f16(w["d"])[:, (width * j) // 256][:, None]
        q = w["codes"][:, inside]
        if fmt == synth.Q6_K:
            want = 3 * d * (q - 32.0)
        elif fmt == synth.IQ4_XS:
            want = 3 * d * np.array(CODEBOOK, float)[q]
        else:
            want = 3 * d * q
        assert np.array_equal(got[:, inside], want)


@pytest.mark.parametrize("fmt", synth.KQUANTS)
def test_super_block_scale_covers_256_columns(fmt):
    """Doubling d of super-block s doubles exactly columns [256 s, 256 s + 256)."""
    w = synth.kquant_weights(synth.rng(21), fmt, 3, 1024)
    base = oracle.ops.dequant(w)
    w2 = dict(w)
    w2["d"] = w["d"].copy()
    d = oracle.decode_f16(w["d"][:, 2])
    w2["d"][:, 2] = synth.to_f16_bits(2 * d)
    if fmt in (synth.Q4_K, synth.Q5_K):
        w["mins"][:] = 0
        base = oracle.ops.dequant(w)
        w2["mins"] = w["mins"]
    got = oracle.ops.dequant(w2)
    cols = np.arange(1024)
    inside = (cols >= 512) & (cols < 768)
    assert np.array_equal(got[:, ~inside], base[:, ~inside])
    assert np.array_equal(got[:, inside], 2 * base[:, inside])


def test_iq4_xs_codebook_and_scale_offset():
    """ls = 33 and d = 1 give the codebook entry itself; ls = 32 gives zero."""
    n, k = 16, 256
    w = {"fmt": synth.IQ4_XS, "codes": np.tile(np.arange(16, dtype=np.uint8), (n, k // 16)),
         "d": synth.to_f16_bits(np.ones((n, 1))), "sub": np.full((n, k // 32), 33, np.uint8)}
    got = oracle.ops.dequant(w)
    assert np.array_equal(got[0, :16], np.array(CODEBOOK, float))
    w["sub"][:] = 32
    assert (oracle.ops.dequant(w) == 0).all()
    assert all(a < b for a, b in zip(CODEBOOK, CODEBOOK[1:])) and -128 <= min(CODEBOOK) and max(CODEBOOK) <= 127


def test_gemv_a8_equals_the_w4a8_integer_form():
    """Q4_K with (sc, m, dmin) = (1, 8, d) is Q4_0: its Q8_0-activation GEMV
    equals the W4A8 oracle's integer block-dot form (a separate formulation)."""
    g = synth.rng(22)
    w = synth.kquant_weights(g, synth.Q4_K, 8, 1024)
    w["sub"][:] = 1
    w["mins"][:] = 8
    w["dmin"] = w["d"].copy()
    q40 = {"fmt": "q4_0", "codes": w["codes"], "scales": np.repeat(w["d"], 8, axis=1)}
    xq, xd, _ = oracle.quantize_q8_0_act(synth.x_f32(synth.rng(23), 3, 1024))
    a = oracle.gemv_a8(w, xq, xd)
    b = oracle.gemv_q4_0_a8(q40, xq, xd)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)


def test_generator_ranges():
    for fmt, hi in ((synth.Q4_K, 15), (synth.Q5_K, 31), (synth.Q6_K, 63), (synth.IQ4_XS, 15)):
        w = synth.kquant_weights(synth.rng(24), fmt, 64, 512)
        assert w["codes"].max() == hi and w["codes"].min() == 0
        assert w["d"].shape == (64, 2)
        if fmt == synth.Q6_K:
            assert w["sub"].dtype == np.int8 and w["sub"].shape == (64, 32)
        else:
            assert w["sub"].max() <= 63 and w["sub"].shape == (64, 16)
