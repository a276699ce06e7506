"""GPU parity of the MoE prefill path (moe_prefill: routing, expert-major
grouping, grouped gate/up + SwiGLU and down GEMMs on the matrix cores,
combine) against the oracle, stage by stage as for the decode path, plus
token independence, determinism and the 35B-A3B-like layer at 512 tokens."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.gpu_util import assert_within, dev, empty, host, require_gpu
from tests.test_gpu_moe import Layer, read_workspace

pytestmark = pytest.mark.gpu


def run_prefill(layer: Layer, x_bits, logits):
    import torch

    L = layer.L
    t = x_bits.shape[0]
    d = layer.desc()
    nbytes = qg.moe_prefill_workspace_bytes(d, t)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y = empty((t, L.hidden), torch.float32)
    qg.moe_prefill(d, dev(x_bits), dev(logits), t, y, ws)
    return host(y), host(ws)


def routing_from_ws(wsh, L, t):
    P = t * (L.top_k + int(L.has_shared))
    off = 0
    for nb in (4, 4 * P, 4 * (P + 1), 4 * P, 4 * P, 2 * P * L.inter, 4 * P * 2 * L.inter, 4 * P * L.hidden):
        off = (off + nb + 255) // 256 * 256
    ids = wsh[off:off + 4 * t * L.top_k].view(np.int32).reshape(t, L.top_k)
    off = (off + 4 * t * L.top_k + 255) // 256 * 256
    wts = wsh[off:off + 4 * t * L.top_k].view(np.float32).reshape(t, L.top_k)
    return ids, wts


def check_prefill(L: synth.MoELayer, layer: Layer):
    t = L.x.shape[0]
    y, wsh = run_prefill(layer, L.x, L.logits)
    ids, wts = routing_from_ws(wsh, L, t)
    rid, _ = oracle.route_topk(L.logits, L.top_k)
    assert np.array_equal(ids, rid)
    W = read_workspace(wsh, L, t)
    csr = oracle.group_by_expert(ids, L.n_experts, L.has_shared)
    assert W["n_groups"] == len(csr["experts"])
    for key in ("experts", "offsets", "tok", "slot"):
        assert np.array_equal(W[key], csr[key]), key
    # stage 1: gate/up per pair (matrix-core products, fp32 accumulation)
    assert_within(W["h"], oracle.ops.moe_gate_up(L, L.x, csr), oracle.ops.moe_gate_up_abs(L, L.x, csr), "h")
    # stage 2: SwiGLU from the GPU's h, within one bf16 ulp
    exact = oracle.swiglu(W["h"].astype(np.float64))
    assert np.all(np.abs(oracle.decode_bf16(W["a"]) - exact) <= oracle.bf16_ulp(exact))
    # stage 3: down per pair from the GPU's a
    o_ref = oracle.ops.moe_down(L, W["a"], csr)
    o_abs = oracle.ops.moe_down(L, W["a"], csr, absolute=True)
    assert_within(W["o"], o_ref, o_abs, "o")
    # stage 4: weighted combine (GPU routing weights) over the exact o
    y_ref = oracle.ops.moe_combine(o_ref, wts, csr, t, L.top_k)
    y_abs = oracle.ops.moe_combine(o_abs, np.abs(wts), csr, t, L.top_k)
    assert_within(y, y_ref, y_abs, "y")
    return y


@pytest.mark.parametrize("t,E,k,H,I,shared", [(1, 4, 2, 512, 512, True), (17, 8, 2, 512, 512, True),
                                              (40, 64, 8, 1024, 512, False), (33, 16, 8, 512, 1024, True),
                                              (100, 256, 8, 2048, 512, True), (70, 5, 4, 2048, 2048, False)])
def test_moe_prefill_small(t, E, k, H, I, shared):
    require_gpu()
    print(f"[moe prefill t={t} E={E} k={k} H={H} I={I} shared={shared}]", flush=True)
    L = synth.moe_case(t=t, n_experts=E, top_k=k, hidden=H, inter=I, has_shared=shared, seed=t * 7 + E)
    check_prefill(L, Layer(L))


def test_moe_prefill_tokens_are_independent_and_deterministic():
    """A token's output does not depend on the other tokens of the call (they
    change which tiles its pairs share), and repeated calls are bitwise equal."""
    require_gpu()
    L = synth.moe_case(t=48, n_experts=16, top_k=4, hidden=512, inter=512, has_shared=True, seed=3)
    layer = Layer(L)
    y, _ = run_prefill(layer, L.x, L.logits)
    y2, _ = run_prefill(layer, L.x, L.logits)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    for lo, hi in ((0, 1), (5, 17), (40, 48)):
        ys, _ = run_prefill(layer, L.x[lo:hi], L.logits[lo:hi])
        assert np.array_equal(ys.view(np.uint32), y[lo:hi].view(np.uint32))


def test_moe_prefill_half_row_blocks():
    """384 tokens over 128 experts (H=1024, K = 1024 for gate/up): on a
    256-CU part each XCD's gate/up items leave a last round under half full,
    which runs as half row blocks.  Every output against the oracle, and
    token slices (other tilings, no half blocks) bitwise equal."""
    require_gpu()
    print("[moe prefill half row blocks t=384]", flush=True)
    L = synth.moe_case(t=384, n_experts=128, top_k=8, hidden=1024, inter=512, has_shared=True, seed=384)
    layer = Layer(L)
    y = check_prefill(L, layer)
    for lo, hi in ((0, 64), (300, 384)):
        ys, _ = run_prefill(layer, L.x[lo:hi], L.logits[lo:hi])
        assert np.array_equal(ys.view(np.uint32), y[lo:hi].view(np.uint32)), (lo, hi)


def test_moe_prefill_unsupported_shapes():
    require_gpu()
    L = synth.moe_case(t=2, n_experts=4, top_k=2, hidden=256, inter=64, has_shared=False, seed=1)
    d = Layer(L).desc()
    assert qg.moe_prefill_workspace_bytes(d, 2) == 0  # hidden 256: not a supported tile size


def test_moe_prefill_full_layer_512_tokens():
    """The 35B-A3B-like layer (256 + 1 experts, H=2048, I=512, top-8) at 512
    tokens: every expert active."""
    require_gpu()
    print("[moe prefill full layer t=512]", flush=True)
    base = synth.moe_case(t=4)
    g = synth.rng(synth.seed_for(7, 99))
    t = 512
    L = synth.MoELayer(base.n_experts, base.top_k, base.hidden, base.inter, base.has_shared,
                       gate_up=base.gate_up, down=base.down, x=synth.x_bf16(g, t, base.hidden),
                       logits=synth.logits_f32(g, t, base.n_experts))
    check_prefill(L, Layer(L))
