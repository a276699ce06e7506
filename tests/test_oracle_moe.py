"""Pins of the oracle's router, expert grouping, SwiGLU, MoE chain and prefill
GEMM (CPU only)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.conftest import load_golden

pytestmark = pytest.mark.cpu


def _route_ex(id_):
    return next(e for e in load_golden("routing_examples.json")["examples"] if e["id"] == id_)


def test_ex5_router_tie_to_lower_index():
    e = _route_ex("EX-5")
    ids, w = oracle.route_topk(np.array(e["logits"], np.float32), e["top_k"])
    assert ids.tolist() == e["ids"]
    assert np.allclose(w, e["weights"], rtol=1e-15, atol=0)
    assert w[0, 0] == pytest.approx(1 / (1 + math.exp(-2)), rel=1e-15)


def test_ex10_grouping():
    e = _route_ex("EX-10")
    ids, _ = oracle.route_topk(np.array(e["logits"], np.float32), e["top_k"])
    assert ids.tolist() == e["ids"]
    csr = oracle.group_by_expert(ids, e["n_experts"], e["has_shared"])
    for key, val in e["csr"].items():
        assert csr[key].tolist() == val, key


def test_router_against_torch_on_distinct_logits():
    g = synth.rng(41)
    L = synth.logits_f32(g, 6, 256)
    ids, w = oracle.route_topk(L, 8)
    tv, ti = torch.topk(torch.from_numpy(L).double(), 8, dim=1)
    assert np.array_equal(ids, ti.numpy())
    ref = torch.softmax(tv, dim=1).numpy()
    assert np.allclose(w, ref, rtol=1e-14, atol=0)
    # renormalised global softmax gives the same weights
    full = torch.softmax(torch.from_numpy(L).double(), dim=1).numpy()
    sel = np.take_along_axis(full, ids, axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)


def test_router_selection_is_exact_brute_force():
    g = synth.rng(42)
    L = np.round(synth.logits_f32(g, 20, 12) * 2).astype(np.float32) / 2  # many ties
    ids, _ = oracle.route_topk(L, 4)
    for t in range(20):
        key = sorted(range(12), key=lambda j: (Fraction(float(-L[t, j])), j))
        assert ids[t].tolist() == key[:4]


def test_grouping_properties():
    g = synth.rng(43)
    ids, _ = oracle.route_topk(synth.logits_f32(g, 4, 256), 8)
    csr = oracle.group_by_expert(ids, 256, True)
    ex, off = csr["experts"], csr["offsets"]
    assert list(ex[:-1]) == sorted(set(ids.ravel().tolist())) and ex[-1] == 256
    assert off[0] == 0 and off[-1] == len(csr["tok"]) == 4 * 9
    seen = set()
    for u in range(len(ex)):
        pairs = list(zip(csr["tok"][off[u]:off[u + 1]], csr["slot"][off[u]:off[u + 1]]))
        assert pairs == sorted(pairs)
        for t, s in pairs:
            assert (ids[t, s] if s < 8 else 256) == ex[u]
            seen.add((int(t), int(s)))
    assert len(seen) == 36


def test_silu_against_torch_and_closed_forms():
    g = np.linspace(-30, 30, 1001)
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    assert np.allclose(oracle.silu(g), ref, rtol=1e-15, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([-1000.0]))[0] == 0.0
    assert oracle.silu(np.array([1000.0]))[0] == 1000.0


def test_swiglu_gate_is_first_half():
    h = np.array([[0.0, 2.0, 5.0, 7.0]])  # g = [0, 2], u = [5, 7]
    a = oracle.swiglu(h)
    assert a[0, 0] == 0.0
    assert a[0, 1] == pytest.approx(2.0 / (1 + math.exp(-2.0)) * 7.0, rel=1e-15)


def _small_layer(E=4, top_k=2, H=32, I=16, shared=True, seed=44):
    return synth.moe_case(t=3, n_experts=E, top_k=top_k, hidden=H, inter=I, has_shared=shared, seed=seed)


def test_moe_single_expert_equals_dense_chain():
    L = synth.moe_case(t=2, n_experts=1, top_k=1, hidden=32, inter=16, has_shared=False, seed=45)
    ids, w = oracle.route_topk(L.logits, 1)
    assert np.all(ids == 0) and np.all(w == 1.0)
    out = oracle.moe_forward(L, L.x, ids, w)
    h = oracle.gemv(L.gate_up[0], L.x)
    a = oracle.swiglu(h)
    dW = oracle.ops.dequant(L.down[0])
    y = a @ dW.T
    assert np.allclose(out["y"], y, rtol=1e-14, atol=1e-14)


def test_moe_combine_by_hand():
    csr = {"experts": np.array([0, 1, 2]), "offsets": np.array([0, 1, 2, 3]),
           "tok": np.array([0, 0, 0]), "slot": np.array([0, 1, 2])}
    o = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    y = oracle.ops.moe_combine(o, np.array([[0.25, 0.75]]), csr, 1, 2)
    assert y.tolist() == [[0.25 + 7.5 + 100.0, 0.5 + 15.0 + 200.0]]


def test_moe_relabelling_experts_changes_nothing():
    L = _small_layer()
    ids, w = oracle.route_topk(L.logits, L.top_k)
    y0 = oracle.moe_forward(L, L.x, ids, w)["y"]
    perm = np.array([2, 0, 3, 1])  # new label of old expert e is perm[e]
    L2 = _small_layer()
    for e in range(4):
        L2.gate_up[perm[e]] = L.gate_up[e]
        L2.down[perm[e]] = L.down[e]
    logits2 = np.empty_like(L.logits)
    logits2[:, perm] = L.logits
    ids2, w2 = oracle.route_topk(logits2, L.top_k)
    assert np.array_equal(perm[ids], ids2)
    y2 = oracle.moe_forward(L2, L.x, ids2, w2)["y"]
    assert np.allclose(y0, y2, rtol=1e-13, atol=1e-13)


def test_moe_tokens_are_independent():
    # batch invariance of the definition: token t's output ignores other tokens
    L = _small_layer()
    ids, w = oracle.route_topk(L.logits, L.top_k)
    y = oracle.moe_forward(L, L.x, ids, w)["y"]
    for t in range(3):
        yt = oracle.moe_forward(L, L.x[t:t + 1], ids[t:t + 1], w[t:t + 1])["y"]
        assert np.allclose(y[t], yt[0], rtol=1e-14, atol=1e-14)


def test_moe_shared_expert_has_unit_weight():
    L = _small_layer()
    ids, w = oracle.route_topk(L.logits, L.top_k)
    with_sh = oracle.moe_forward(L, L.x, ids, w)
    L.has_shared = False
    without = oracle.moe_forward(L, L.x, ids, w)
    sh = oracle.swiglu(oracle.gemv(L.gate_up[4], L.x)) @ oracle.ops.dequant(L.down[4]).T
    assert np.allclose(with_sh["y"] - without["y"], sh, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- prefill

def test_ex9_prefill():
    ex6 = next(e for e in load_golden("worked_examples.json")["examples"] if e["id"] == "EX-6")
    ex9 = next(e for e in load_golden("worked_examples.json")["examples"] if e["id"] == "EX-9")
    w = {"fmt": "nvfp4", "codes": np.array(ex6["codes"], np.uint8),
         "scales": np.array(ex6["scales"], np.uint8), "tensor_scale": np.float32(ex6["tensor_scale"])}
    X = np.zeros((2, 32), np.float32)
    X[0] = 1.0
    X[1, 20] = 1.0
    Y, _ = oracle.prefill(w, synth.to_bf16_bits(X))
    assert Y.tolist() == ex9["Y"]


def test_prefill_one_hot_rows_give_dequantized_columns():
    g = synth.rng(46)
    w = synth.nvfp4_weights(g, 9, 64, tensor_scale=1.0)
    X = np.zeros((4, 64), np.float32)
    for m, col in enumerate((0, 15, 16, 63)):
        X[m, col] = 1.0
    Y, _ = oracle.prefill(w, synth.to_bf16_bits(X))
    D = oracle.dequant_nvfp4(w)
    for m, col in enumerate((0, 15, 16, 63)):
        assert np.array_equal(Y[m], D[:, col])


def test_prefill_subsets():
    g = synth.rng(47)
    w = synth.nvfp4_weights(g, 12, 32)
    X = synth.x_bf16(g, 5, 32)
    Y, A = oracle.prefill(w, X)
    Ys, As = oracle.prefill(w, X, rows=[1, 4], cols=[0, 7, 11])
    assert np.array_equal(Ys, Y[np.ix_([1, 4], [0, 7, 11])])
    assert np.array_equal(As, A[np.ix_([1, 4], [0, 7, 11])])
