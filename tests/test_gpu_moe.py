"""GPU parity of the MoE decode path: router (exact ids), expert-major CSR
(exact), grouped gate/up + SwiGLU, grouped down and the weighted combine,
checked stage by stage against the oracle; batch invariance; full size."""
import ctypes

import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.conftest import load_golden
from tests.gpu_util import assert_within, dev, dev_u8, empty, host, require_gpu

pytestmark = pytest.mark.gpu


def route_gpu(logits, top_k):
    import torch

    t, e = logits.shape
    ids = empty((t, top_k), torch.int32)
    w = empty((t, top_k), torch.float32)
    qg.moe_route_topk(dev(logits), t, e, top_k, ids, w)
    return ids, w


def test_router_worked_example():
    require_gpu()
    ex = next(e for e in load_golden("routing_examples.json")["examples"] if e["id"] == "EX-5")
    ids, w = route_gpu(np.array(ex["logits"], np.float32), ex["top_k"])
    assert host(ids).tolist() == ex["ids"]
    assert np.allclose(host(w), ex["weights"], rtol=1e-6, atol=0)


@pytest.mark.parametrize("t,e,k", [(1, 256, 8), (4, 256, 8), (16, 256, 8), (3, 60, 4), (2, 1024, 16),
                                   (5, 8, 8), (7, 130, 1)])
def test_router_random(t, e, k):
    require_gpu()
    g = synth.rng(t * 1000 + e + k)
    L = synth.logits_f32(g, t, e)
    L[0, 3] = L[0, 5] = L[0].max()  # an exact tie at the top
    ids, w = route_gpu(L, k)
    rid, rw = oracle.route_topk(L, k)
    assert np.array_equal(host(ids), rid)
    assert np.all(np.abs(host(w) - rw) <= 1e-6 * rw + 1e-9)


def test_router_many_ties():
    require_gpu()
    g = synth.rng(9)
    L = (np.round(synth.logits_f32(g, 8, 64) * 2) / 2).astype(np.float32)
    ids, _ = route_gpu(L, 8)
    assert np.array_equal(host(ids), oracle.route_topk(L, 8)[0])


class Layer:
    """A MoE layer packed on the device, one buffer for all gate_up and one for all down."""

    def __init__(self, L: synth.MoELayer, experts=None):
        import torch

        self.L = L
        E = L.n_experts + (1 if L.has_shared else 0)
        H, I = L.hidden, L.inter
        self.gu_stride = qg.qg_packed_bytes(qg.QG_NVFP4, 2 * I, H)
        self.dn_stride = qg.qg_packed_bytes(qg.QG_NVFP4, H, I)
        gu = np.zeros((E, self.gu_stride), np.uint8)
        dn = np.zeros((E, self.dn_stride), np.uint8)
        for e in range(E):
            if L.gate_up[e] is None:
                continue
            gu[e] = qg.qg_pack_nvfp4_gate_up(L.gate_up[e]["codes"], L.gate_up[e]["scales"])
            dn[e] = qg.qg_pack_nvfp4(L.down[e]["codes"], L.down[e]["scales"])
        self.gu = dev_u8(gu)
        self.dn = dev_u8(dn)
        self.gu_s = torch.full((E,), 0.01, dtype=torch.float32, device="cuda")
        self.dn_s = torch.full((E,), 0.01, dtype=torch.float32, device="cuda")

    def desc(self, flags=qg.QG_MOE_KEEP_H):
        L = self.L
        return qg.QgMoeDesc(n_experts=L.n_experts, top_k=L.top_k, has_shared=int(L.has_shared), flags=flags,
                            hidden=L.hidden, inter=L.inter, gate_up=self.gu.data_ptr(),
                            gate_up_stride=self.gu_stride, down=self.dn.data_ptr(), down_stride=self.dn_stride,
                            gate_up_scale=self.gu_s.data_ptr(), down_scale=self.dn_s.data_ptr())


def run_moe(layer: Layer, x_bits, ids, w):
    import torch

    t = x_bits.shape[0]
    d = layer.desc()
    nbytes = qg.moe_workspace_bytes(d, t)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y = empty((t, layer.L.hidden), torch.float32)
    qg.moe_gemv_grouped(d, dev(x_bits), ids, w, t, y, ws)
    return host(y), host(ws), nbytes


def read_workspace(ws: np.ndarray, L: synth.MoELayer, t: int):
    """Decode the documented workspace layout."""
    P = t * (L.top_k + (1 if L.has_shared else 0))
    H, I = L.hidden, L.inter
    off = 0

    def take(nbytes):
        nonlocal off
        at = off
        off = (off + nbytes + 255) // 256 * 256
        return at

    o_ng, o_ex, o_off = take(4), take(4 * P), take(4 * (P + 1))
    o_tok, o_slot, o_a = take(4 * P), take(4 * P), take(2 * P * I)
    o_h, o_o = take(4 * P * 2 * I), take(4 * P * H)
    i32 = lambda at, cnt: ws[at:at + 4 * cnt].view(np.int32)  # noqa: E731
    ng = int(i32(o_ng, 1)[0])
    return {
        "n_groups": ng,
        "experts": i32(o_ex, ng), "offsets": i32(o_off, ng + 1),
        "tok": i32(o_tok, P), "slot": i32(o_slot, P),
        "a": ws[o_a:o_a + 2 * P * I].view(np.uint16).reshape(P, I),
        "h": ws[o_h:o_h + 4 * P * 2 * I].view(np.float32).reshape(P, 2 * I),
        "o": ws[o_o:o_o + 4 * P * H].view(np.float32).reshape(P, H),
    }


def check_moe(L: synth.MoELayer, layer: Layer, t: int):
    ids_d, w_d = route_gpu(L.logits, L.top_k)
    ids, wts = host(ids_d), host(w_d)
    rid, rw = oracle.route_topk(L.logits, L.top_k)
    assert np.array_equal(ids, rid)
    y, ws, _ = run_moe(layer, L.x, ids_d, w_d)
    W = read_workspace(ws, L, t)
    csr = oracle.group_by_expert(ids, L.n_experts, L.has_shared)
    assert W["n_groups"] == len(csr["experts"])
    for key in ("experts", "offsets", "tok", "slot"):
        assert np.array_equal(W[key], csr[key]), key
    # stage 1: gate/up per pair
    assert_within(W["h"], oracle.ops.moe_gate_up(L, L.x, csr), oracle.ops.moe_gate_up_abs(L, L.x, csr), "moe h")
    # stage 2: SwiGLU from the GPU's h, within one bf16 ulp
    exact = oracle.swiglu(W["h"].astype(np.float64))
    assert np.all(np.abs(oracle.decode_bf16(W["a"]) - exact) <= oracle.bf16_ulp(exact))
    # stage 3: down per pair from the GPU's a
    o_ref = oracle.ops.moe_down(L, W["a"], csr)
    o_abs = oracle.ops.moe_down(L, W["a"], csr, absolute=True)
    assert_within(W["o"], o_ref, o_abs, "moe o")
    # stage 4: weighted combine (GPU weights) over the exact o
    y_ref = oracle.ops.moe_combine(o_ref, wts, csr, t, L.top_k)
    y_abs = oracle.ops.moe_combine(o_abs, np.abs(wts), csr, t, L.top_k)
    assert_within(y, y_ref, y_abs, "moe y")
    return y, ids_d, w_d


@pytest.mark.parametrize("t,E,k,H,I,shared", [(1, 4, 2, 64, 32, True), (3, 8, 3, 96, 64, False),
                                              (4, 16, 8, 512, 128, True), (16, 32, 8, 256, 64, True),
                                              (2, 6, 6, 2048, 512, True), (5, 64, 4, 2080, 96, False),
                                              (1, 16, 4, 2080, 96, True)])
def test_moe_small(t, E, k, H, I, shared):
    require_gpu()
    print(f"[moe t={t} E={E} k={k} H={H} I={I} shared={shared}]", flush=True)
    L = synth.moe_case(t=t, n_experts=E, top_k=k, hidden=H, inter=I, has_shared=shared, seed=t * 100 + E)
    check_moe(L, Layer(L), t)


@pytest.mark.parametrize("t,E,k,H,I,shared", [(2, 16, 4, 4096, 256, True),   # gate/up 2 chunks per lane
                                              (3, 8, 2, 2048, 2048, True),   # down rows over 64 lanes
                                              (2, 8, 2, 2048, 4096, False),  # down 2 chunks per lane
                                              (4, 64, 8, 2048, 512, True),   # up to 4 routed groups per wave
                                              (2, 40, 8, 2048, 512, True),   # 17 groups
                                              (4, 8, 8, 2048, 512, True),    # 8 groups of 4 tokens, one per wave
                                              (3, 4, 4, 2048, 512, True),    # waves 4-7 own no routed group
                                              (2, 3, 2, 1024, 256, False)])  # repeated experts, no shared one
def test_moe_tile_path(t, E, k, H, I, shared):
    """Two to four tokens run the row-tile kernels: every launch shape they
    take, against the oracle."""
    require_gpu()
    print(f"[moe tile t={t} E={E} k={k} H={H} I={I} shared={shared}]", flush=True)
    L = synth.moe_case(t=t, n_experts=E, top_k=k, hidden=H, inter=I, has_shared=shared, seed=t * 1000 + E + H)
    check_moe(L, Layer(L), t)


def test_moe_tile_path_batch_invariance():
    """Token rows of a 4-token call (row-tile kernels) equal the same tokens
    run alone (per-group kernels) bitwise, at the full layer width."""
    require_gpu()
    L = synth.moe_case(t=4, n_experts=32, top_k=8, hidden=2048, inter=512, has_shared=True, seed=91)
    layer = Layer(L)
    ids_d, w_d = route_gpu(L.logits, 8)
    y4, _, _ = run_moe(layer, L.x, ids_d, w_d)
    for t in range(4):
        y1, _, _ = run_moe(layer, L.x[t:t + 1], ids_d[t:t + 1].contiguous(), w_d[t:t + 1].contiguous())
        assert np.array_equal(y1.view(np.uint32), y4[t:t + 1].view(np.uint32)), t
    for t in (2, 3):  # 2- and 3-token prefixes, also on the row-tile kernels
        yt, _, _ = run_moe(layer, L.x[:t], ids_d[:t].contiguous(), w_d[:t].contiguous())
        assert np.array_equal(yt.view(np.uint32), y4[:t].view(np.uint32)), t


def test_moe_single_expert_matches_dense_kernels():
    """E=1, top-1, no shared expert: the grouped path equals the dense
    gate+up/SwiGLU and down kernels bitwise."""
    import torch

    require_gpu()
    L = synth.moe_case(t=3, n_experts=1, top_k=1, hidden=2048, inter=512, has_shared=False, seed=5)
    layer = Layer(L)
    ids_d, w_d = route_gpu(L.logits, 1)
    y, _, _ = run_moe(layer, L.x, ids_d, w_d)
    from tests.gpu_util import pack_dev, pack_dev_gate_up
    a = empty((3, 512), torch.int16)
    qg.qgemv_nvfp4_swiglu(pack_dev_gate_up(L.gate_up[0]), 0.01, 512, 2048, dev(L.x), 3, a, None)
    yd = empty((3, 2048), torch.float32)
    qg.qgemv_nvfp4(pack_dev(L.down[0]), 0.01, 2048, 512, a, 3, yd)
    # weight 1.0: fmaf(1, o, 0) == o
    assert np.array_equal(y.view(np.uint32), host(yd).view(np.uint32))


def test_moe_batch_invariance_and_determinism():
    require_gpu()
    L = synth.moe_case(t=4, n_experts=32, top_k=8, hidden=512, inter=128, has_shared=True, seed=77)
    layer = Layer(L)
    ids_d, w_d = route_gpu(L.logits, 8)
    y4, _, _ = run_moe(layer, L.x, ids_d, w_d)
    for _ in range(5):
        assert np.array_equal(run_moe(layer, L.x, ids_d, w_d)[0].view(np.uint32), y4.view(np.uint32))
    for t in range(4):
        y1, _, _ = run_moe(layer, L.x[t:t + 1], ids_d[t:t + 1].contiguous(), w_d[t:t + 1].contiguous())
        assert np.array_equal(y1.view(np.uint32), y4[t:t + 1].view(np.uint32)), t


@pytest.mark.parametrize("t,E,k,shared,H,I", [(1, 256, 8, True, 256, 64), (4, 64, 8, True, 256, 64),
                                              (16, 300, 8, False, 256, 64), (3, 8, 2, True, 256, 64),
                                              (4, 128, 8, True, 2048, 512), (2, 300, 8, False, 2048, 256),
                                              (1, 300, 8, False, 256, 64), (1, 8, 2, True, 256, 64),
                                              (4, 8, 8, True, 2048, 512), (3, 4, 4, True, 2048, 512),
                                              (1, 64, 1, True, 2080, 96), (1, 16, 4, True, 2080, 96)])
def test_moe_forward_matches_route_then_grouped(t, E, k, shared, H, I):
    """The fused path (routing inside the gate/up kernel) gives bitwise the
    same ids, weights and outputs as moe_route_topk + moe_gemv_grouped, and
    publishes the oracle's expert-major grouping (at t = 1 it is built
    directly from the routing wave)."""
    import torch

    require_gpu()
    L = synth.moe_case(t=t, n_experts=E, top_k=k, hidden=H, inter=I, has_shared=shared, seed=E + t)
    layer = Layer(L)
    ids_d, w_d = route_gpu(L.logits, k)
    y_split, _, _ = run_moe(layer, L.x, ids_d, w_d)
    d = layer.desc()
    nbytes = qg.moe_workspace_bytes(d, t)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y = empty((t, L.hidden), torch.float32)
    qg.moe_forward(d, dev(L.x), dev(L.logits), t, y, ws)
    assert np.array_equal(host(y).view(np.uint32), y_split.view(np.uint32))
    # the routing it wrote sits at the end of the workspace
    wsh = host(ws)
    P = t * (k + int(shared))
    off = 0
    for nb in (4, 4 * P, 4 * (P + 1), 4 * P, 4 * P, 2 * P * I, 4 * P * 2 * I, 4 * P * H):
        off = (off + nb + 255) // 256 * 256
    ids = wsh[off:off + 4 * t * k].view(np.int32).reshape(t, k)
    off = (off + 4 * t * k + 255) // 256 * 256
    wts = wsh[off:off + 4 * t * k].view(np.float32).reshape(t, k)
    assert np.array_equal(ids, host(ids_d)) and np.array_equal(wts.view(np.uint32), host(w_d).view(np.uint32))
    W = read_workspace(wsh, L, t)
    csr = oracle.group_by_expert(ids, E, shared)
    assert W["n_groups"] == len(csr["experts"])
    for key in ("experts", "offsets", "tok", "slot"):
        assert np.array_equal(W[key], csr[key]), key


@pytest.fixture(scope="module")
def full_layer():
    """The 35B-A3B-like layer: 256 routed experts + 1 shared, H=2048, I=512."""
    require_gpu()
    print("[moe full layer: generating 257 experts]", flush=True)
    return synth.moe_case(t=4)


@pytest.mark.parametrize("t", [1, 4])
def test_moe_full_size(full_layer, t):
    require_gpu()
    print(f"[moe full t={t}]", flush=True)
    L = synth.MoELayer(full_layer.n_experts, full_layer.top_k, full_layer.hidden, full_layer.inter,
                       full_layer.has_shared, gate_up=full_layer.gate_up, down=full_layer.down,
                       x=full_layer.x[:t], logits=full_layer.logits[:t])
    check_moe(L, Layer(L), t)
