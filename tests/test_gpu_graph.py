"""HIP-graph capture of every device entry point.

The entry points are stream-ordered and allocate nothing, so a caller can
capture them into a graph (the memra and bw24 READMEs decode from graph
replays; the benchmark times its steps that way).  Each case here runs the
calls eagerly once, captures the same calls into a graph, and replays the
graph several times with other work of the program (eager library calls on
other inputs, torch work, synchronisations) in between.  Before every replay
the outputs are overwritten with garbage; after it they must equal the eager
results bit for bit.
"""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import synth
from tests.gpu_util import KQ_FMT, dev, empty, host, pack_dev, pack_dev_gate_up, require_gpu
from tests.test_gpu_moe import Layer

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _check_graph(name, run, outputs, interleave):
    """run(): enqueue the calls on the current stream; outputs: device
    tensors they write; interleave(i): other eager work between replays."""
    import torch

    print(f"[graph {name}]", flush=True)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run()
    torch.cuda.synchronize()
    ref = [host(o).view(np.uint8).copy() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o in outputs:
            o.view(torch.uint8).fill_(0xA5 + i)
        interleave(i)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for j, o in enumerate(outputs):
            got = host(o).view(np.uint8)
            assert np.array_equal(got, ref[j]), f"{name}: replay {i}, output {j} differs from the eager result"


def _noise():
    """Eager torch work that touches the device caches between replays."""
    import torch

    a = torch.randn(1 << 20, device="cuda")
    return float((a * 2).sum())


@pytest.mark.parametrize("m", [1, 3])
def test_graph_dense_mlp(m):
    """gate+up + SwiGLU then down, NVFP4; the down rows (6144) take the
    LDS-staged batch-1 kernel at m = 1."""
    import torch

    require_gpu()
    g = synth.rng(500 + m)
    H, I = 2048, 6144
    gu = synth.nvfp4_weights(g, 2 * I, H)
    dn = synth.nvfp4_weights(g, H, I)
    wgu, wdn = pack_dev_gate_up(gu), pack_dev(dn)
    x = dev(synth.x_bf16(g, m, H))
    x_other = dev(synth.x_bf16(g, m, H))
    a = empty((m, I), torch.int16)
    y = empty((m, H), torch.float32)
    a2 = empty((m, I), torch.int16)

    def run():
        qg.qgemv_nvfp4_swiglu(wgu, 0.01, I, H, x, m, a)
        qg.qgemv_nvfp4(wdn, 0.01, H, I, a, m, y)

    def interleave(i):
        qg.qgemv_nvfp4_swiglu(wgu, 0.01, I, H, x_other, m, a2)
        _noise()

    _check_graph(f"dense m={m}", run, [a, y], interleave)


@pytest.mark.parametrize("m", [1, 4])
def test_graph_w4a8(m):
    """Q8_0 activation quantizer then the Q4_0 x Q8_0 GEMV."""
    import torch

    require_gpu()
    g = synth.rng(600 + m)
    n, k = 777, 5120
    w = pack_dev(synth.q4_0_weights(g, n, k))
    x = dev(synth.x_f32(g, m, k))
    xq = empty((m, k), torch.int8)
    xd = empty((m, k // 32), torch.int16)
    xs = empty((m, k // 32), torch.int32)
    y = empty((m, n), torch.float32)

    def run():
        qg.qg_quantize_q8_0_act(x, m, k, xq, xd, xs)
        qg.qgemv_q4_0_a8(w, n, k, xq, xd, xs, m, y)

    _check_graph(f"w4a8 m={m}", run, [xq, xd, xs, y], lambda i: _noise())


@pytest.mark.parametrize("fmt", ["q4_k", "iq4_xs"])
def test_graph_kquant(fmt):
    import torch

    require_gpu()
    g = synth.rng(700)
    n, k, m = 300, 2048, 2
    w = pack_dev(synth.kquant_weights(g, fmt, n, k))
    x = dev(synth.x_f32(g, m, k))
    xq = empty((m, k), torch.int8)
    xd = empty((m, k // 32), torch.int16)
    xs = empty((m, k // 32), torch.int32)
    y = empty((m, n), torch.float32)

    def run():
        qg.qg_quantize_q8_0_act(x, m, k, xq, xd, xs)
        qg.qgemv_kquant_a8(KQ_FMT[fmt], w, n, k, xq, xd, xs, m, y)

    _check_graph(fmt, run, [y], lambda i: _noise())


def test_graph_fp8_and_q8():
    import torch

    require_gpu()
    g = synth.rng(800)
    wf = synth.fp8_weights(g, 500, 4096)
    wq = synth.q8_0_weights(g, 256, 1024)
    from tests.gpu_util import fp8_fmt

    wfd, wqd = pack_dev(wf), pack_dev(wq)
    xb = dev(synth.x_bf16(g, 1, 4096))
    xf = dev(synth.x_f32(g, 1, 1024))
    yf = empty((1, 500), torch.float32)
    yq = empty((1, 256), torch.float32)

    def run():
        qg.qgemv_fp8(fp8_fmt(wf), wfd, 500, 4096, xb, 1, yf)
        qg.qgemv_q8_0(wqd, 256, 1024, xf, 1, yq)

    _check_graph("fp8 + q8_0", run, [yf, yq], lambda i: _noise())


@pytest.mark.parametrize("t", [1, 3])
def test_graph_moe_forward(t):
    """Routing, grouping, gate/up + SwiGLU, down and combine (moe_forward)."""
    import torch

    require_gpu()
    L = synth.moe_case(t=t, n_experts=64, top_k=8, hidden=1024, inter=512, has_shared=True, seed=900 + t)
    layer = Layer(L)
    d = layer.desc()
    nbytes = qg.moe_workspace_bytes(d, t)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ws_other = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    x, logits = dev(L.x), dev(L.logits)
    logits_other = dev(synth.logits_f32(synth.rng(901 + t), t, L.n_experts))
    y = empty((t, L.hidden), torch.float32)
    y_other = empty((t, L.hidden), torch.float32)

    def run():
        qg.moe_forward(d, x, logits, t, y, ws)

    def interleave(i):
        qg.moe_forward(d, x, logits_other, t, y_other, ws_other)
        _noise()

    _check_graph(f"moe_forward t={t}", run, [y], interleave)


def test_graph_moe_prefill():
    import torch

    require_gpu()
    t = 40
    L = synth.moe_case(t=t, n_experts=32, top_k=4, hidden=1024, inter=512, has_shared=True, seed=950)
    layer = Layer(L)
    d = layer.desc()
    nbytes = qg.moe_prefill_workspace_bytes(d, t)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    x, logits = dev(L.x), dev(L.logits)
    y = empty((t, L.hidden), torch.float32)

    def run():
        qg.moe_prefill(d, x, logits, t, y, ws)

    _check_graph("moe_prefill t=40", run, [y], lambda i: _noise())


@pytest.mark.parametrize("m,use_ws", [(64, True), (200, False), (48, False)])
def test_graph_prefill(m, use_ws):
    import torch

    require_gpu()
    g = synth.rng(1000 + m)
    n, k = 768, 4096
    w = pack_dev(synth.nvfp4_weights(g, n, k))
    x = dev(synth.x_bf16(g, m, k))
    y = empty((m, n), torch.int16)
    ws = None
    if use_ws:
        ws = torch.zeros(qg.qgemm_prefill_workspace_bytes(n, k, m), dtype=torch.uint8, device="cuda")

    def run():
        if use_ws:
            qg.qgemm_prefill_ws(w, 0.01, n, k, x, m, y, ws)
        else:
            qg.qgemm_prefill(w, 0.01, n, k, x, m, y)

    _check_graph(f"prefill m={m} ws={use_ws}", run, [y], lambda i: _noise())


def test_graph_prefill_a8():
    import torch

    require_gpu()
    g = synth.rng(1100)
    n, k, m = 384, 2048, 100
    w = pack_dev(synth.q4_0_weights(g, n, k))
    x = dev(synth.x_f32(g, m, k))
    xq = empty((m, k), torch.int8)
    xd = empty((m, k // 32), torch.int16)
    y = empty((m, n), torch.float32)

    def run():
        qg.qg_quantize_q8_0_act(x, m, k, xq, xd, None)
        qg.qgemm_prefill_a8(w, n, k, xq, xd, m, y)

    _check_graph("prefill a8 m=100", run, [y], lambda i: _noise())
