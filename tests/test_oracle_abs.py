"""Pins of the oracle's tolerance scales (CPU only).

Every parity test allows |y_gpu - y_ref| <= 1e-5 * S + 1e-6 per output, with
S = sum_k |w_k * x_k| (the north-star tolerance; the pages' gate is "every
quant kernel against a CPU reference", bw24 and memra READMEs, correctness
gates).  The oracle computes S with helpers of its own (``gemv_abs``,
``gemv_a8_abs``, ``gemv_q4_0_a8_abs``, ``moe_gate_up_abs``,
``moe_down(absolute=True)``, the second output of ``prefill``) and the bf16
output allowance with ``bf16_ulp``.  A mistake that inflated any of them would
loosen every test that uses it without failing one, so each is checked here
against an exact rational brute force that decodes every weight on its own
(independent E4M3 / binary16 decoders, the OCP E2M1 table, int codes) and
sums |w_k * x_k| term by term.  Inputs carry negative weights and negative
activations, so an absolute value dropped on either side changes S.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.test_oracle_gemv import E2M1, _e4m3_fraction, _f16_fraction, _x_fractions
from tests.test_oracle_kquants import brute_value as kq_value
from tests.test_oracle_kquants import f16_fraction as kq_f16

pytestmark = pytest.mark.cpu


def _w_fraction(w: dict, r: int, c: int) -> Fraction:
    """One weight of a dense format, straight from its definition."""
    fmt = w["fmt"]
    if fmt == "nvfp4":
        st = Fraction(float(np.float32(w["tensor_scale"])))
        return E2M1[int(w["codes"][r, c])] * _e4m3_fraction(int(w["scales"][r][c // 16])) * st
    if fmt == "q8_0":
        return _f16_fraction(int(w["scales"][r][c // 32])) * int(w["codes"][r, c])
    if fmt == "q4_0":
        return _f16_fraction(int(w["scales"][r][c // 32])) * (int(w["codes"][r, c]) - 8)
    return kq_value(w, r, c)


def _abs_sum(w: dict, xrow, r: int) -> Fraction:
    return sum(abs(_w_fraction(w, r, c) * xrow[c]) for c in range(len(xrow)))


def _close(got: float, exact: Fraction) -> bool:
    """fp64 sum of at most a few hundred non-negative exact terms: relative error
    far below 2^-40 (an error of the magnitude a bug makes is >= 2^-8)."""
    return abs(Fraction(float(got)) - exact) <= exact * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 100)


def _xhat_fractions(xq, xd):
    """Dequantized Q8_0 activations d_x * q_x as rationals."""
    m, k = xq.shape
    return [[_f16_fraction(int(xd[t, c // 32])) * int(xq[t, c]) for c in range(k)] for t in range(m)]


@pytest.mark.parametrize("fmt,n,k,m", [("nvfp4", 3, 32, 2), ("nvfp4", 5, 64, 1), ("q8_0", 4, 64, 2),
                                       ("q4_0", 3, 96, 3)])
def test_gemv_abs_vs_exact(fmt, n, k, m):
    g = synth.rng(5100 + n + k + m)
    w = {"nvfp4": synth.nvfp4_weights, "q8_0": synth.q8_0_weights, "q4_0": synth.q4_0_weights}[fmt](g, n, k)
    x = synth.x_bf16(g, m, k) if fmt == "nvfp4" else synth.x_f32(g, m, k)
    got = oracle.gemv_abs(w, x)
    X = _x_fractions(x)
    for t in range(m):
        for r in range(n):
            assert _close(got[t, r], _abs_sum(w, X[t], r)), (fmt, t, r)
    rows = [n - 1, 0]
    assert np.array_equal(oracle.gemv_abs(w, x, rows), got[:, rows])


def test_gemv_abs_is_larger_than_the_signed_sum():
    """Cancellation: |sum w x| can be far below sum |w x|; the helper must
    report the latter (here the signed sum is exactly 0)."""
    w = {"fmt": "q8_0", "codes": np.zeros((1, 32), np.int8), "scales": np.full((1, 1), 0x3C00, np.uint16)}
    w["codes"][0, :16], w["codes"][0, 16:] = 3, -3
    x = np.ones((1, 32), np.float32)
    assert oracle.gemv(w, x)[0, 0] == 0.0
    assert oracle.gemv_abs(w, x)[0, 0] == 96.0


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", synth.Q4_K, synth.Q6_K, synth.IQ4_XS])
def test_gemv_a8_abs_vs_exact(fmt):
    g = synth.rng(5200 + len(fmt))
    k = 256
    if fmt in ("q4_0", "q8_0"):
        w = (synth.q4_0_weights if fmt == "q4_0" else synth.q8_0_weights)(g, 3, k)
    else:
        w = synth.kquant_weights(g, fmt, 3, k)
    xq, xd, _ = oracle.quantize_q8_0_act(synth.x_f32(g, 2, k))
    got = oracle.gemv_a8_abs(w, xq, xd)
    X = _xhat_fractions(xq, xd)
    for t in range(2):
        for r in range(3):
            assert _close(got[t, r], _abs_sum(w, X[t], r)), (fmt, t, r)


def test_gemv_q4_0_a8_abs_vs_exact():
    g = synth.rng(5300)
    w = synth.q4_0_weights(g, 4, 128)
    xq, xd, _ = oracle.quantize_q8_0_act(synth.x_f32(g, 3, 128))
    got = oracle.gemv_q4_0_a8_abs(w, xq, xd)
    X = _xhat_fractions(xq, xd)
    for t in range(3):
        for r in range(4):
            assert _close(got[t, r], _abs_sum(w, X[t], r)), (t, r)
    # the integer-form helper and the generic one are the same quantity
    assert np.allclose(got, oracle.gemv_a8_abs(w, xq, xd), rtol=1e-15, atol=0)


def _moe_layer():
    return synth.moe_case(t=3, n_experts=4, top_k=2, hidden=32, inter=32, has_shared=True, seed=5400)


def test_moe_gate_up_abs_vs_exact():
    L = _moe_layer()
    ids, _ = oracle.route_topk(L.logits, L.top_k)
    csr = oracle.group_by_expert(ids, L.n_experts, L.has_shared)
    got = oracle.ops.moe_gate_up_abs(L, L.x, csr)
    X = _x_fractions(L.x)
    for p in range(len(csr["tok"])):
        u = int(np.searchsorted(csr["offsets"], p, side="right")) - 1
        e, t = int(csr["experts"][u]), int(csr["tok"][p])
        for r in range(2 * L.inter):
            assert _close(got[p, r], _abs_sum(L.gate_up[e], X[t], r)), (p, r)


def test_moe_down_abs_vs_exact():
    L = _moe_layer()
    ids, _ = oracle.route_topk(L.logits, L.top_k)
    csr = oracle.group_by_expert(ids, L.n_experts, L.has_shared)
    P = len(csr["tok"])
    a = synth.x_bf16(synth.rng(5401), P, L.inter)  # stands in for the GPU's SwiGLU outputs
    got = oracle.ops.moe_down(L, a, csr, absolute=True)
    A = _x_fractions(a)
    for p in range(P):
        u = int(np.searchsorted(csr["offsets"], p, side="right")) - 1
        e = int(csr["experts"][u])
        for r in range(L.hidden):
            assert _close(got[p, r], _abs_sum(L.down[e], A[p], r)), (p, r)


def test_prefill_abs_vs_exact():
    g = synth.rng(5500)
    w = synth.nvfp4_weights(g, 5, 64)
    X = synth.x_bf16(g, 3, 64)
    _, got = oracle.prefill(w, X)
    Xf = _x_fractions(X)
    for t in range(3):
        for r in range(5):
            assert _close(got[t, r], _abs_sum(w, Xf[t], r)), (t, r)
    _, sub = oracle.prefill(w, X, rows=[2, 0], cols=[4, 1])
    assert np.array_equal(sub, got[np.ix_([2, 0], [4, 1])])


def _bf16_spacing(v: float) -> float:
    """Gap between the two bf16 numbers around |v|, from torch's bf16 nextafter:
    for |v| in [2^(e-1), 2^e) every bf16 number there is 2^(e-8) apart."""
    a = torch.tensor([abs(v)], dtype=torch.float64)
    lo = a.to(torch.bfloat16)
    if lo.double() > a:  # rounded up: step down to the bf16 number below |v|
        lo = torch.nextafter(lo, torch.tensor([0.0], dtype=torch.bfloat16))
    hi = torch.nextafter(lo, torch.tensor([float("inf")], dtype=torch.bfloat16))
    return float(hi.double() - lo.double())


def test_bf16_ulp_vs_torch_spacing():
    g = synth.rng(5600)
    vals = np.concatenate([g.standard_normal(200) * 10.0 ** g.integers(-30, 30, 200),
                           [1.0, 2.0, 0.5, 3.0, -7.75, 1e-38, 2.0 ** -126]])
    for v in vals:
        assert oracle.bf16_ulp(np.array([v]))[0] == _bf16_spacing(float(v)), v


def test_kquant_brute_value_decoder_is_independent():
    """The K-quant brute force used above decodes fp16 by bit fields, not numpy."""
    for bits in (0x0001, 0x03FF, 0x0400, 0x3C00, 0xBC00, 0x7BFF):
        assert float(kq_f16(bits)) == float(np.uint16(bits).view(np.float16))
