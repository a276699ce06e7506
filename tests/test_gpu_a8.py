"""GPU parity of the W4A8 path: the activation quantizer (bit-exact) and the
Q4_0 x Q8_0 integer-dot GEMV."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.conftest import load_golden
from tests.gpu_util import assert_within, dev, empty, host, pack_dev, require_gpu

pytestmark = pytest.mark.gpu


def quantize_gpu(x):
    import torch

    m, k = x.shape
    xq = empty((m, k), torch.int8)
    xd = empty((m, k // 32), torch.int16)
    xs = empty((m, k // 32), torch.int32)
    qg.qg_quantize_q8_0_act(dev(x), m, k, xq, xd, xs)
    return xq, xd, xs


def run_a8(w, xq, xd, xs):
    import torch

    n, k = w["codes"].shape
    m = xq.shape[0]
    y = empty((m, n), torch.float32)
    qg.qgemv_q4_0_a8(pack_dev(w), n, k, xq, xd, xs, m, y)
    return host(y)


def _check_quant(x):
    xq, xd, xs = quantize_gpu(x)
    rq, rd, rs = oracle.quantize_q8_0_act(x)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xd).view(np.uint16), rd)
    assert np.array_equal(host(xs), rs)


def test_quantizer_worked_example():
    require_gpu()
    e = next(e for e in load_golden("worked_examples.json")["examples"] if e["id"] == "EX-4")
    xq, xd, xs = quantize_gpu(np.ones((1, 32), np.float32))
    assert np.all(host(xq) == 127)
    assert int(host(xd).view(np.uint16)[0, 0]) == e["xd_bits"]
    assert int(host(xs)[0, 0]) == e["xs"]


@pytest.mark.parametrize("scale", [1.0, 1e-3, 300.0, 1e-36])
def test_quantizer_bit_exact(scale):
    require_gpu()
    g = synth.rng(int(abs(np.log10(scale))) + 11)
    x = (synth.x_f32(g, 7, 5120) * np.float32(scale)).astype(np.float32)
    x[2, 64:96] = 0.0                    # zero block
    x[3, 0:32] = np.float32(scale)       # constant block
    x[4, 40] = -np.float32(scale) * 9    # lone outlier
    _check_quant(x)


def test_quantizer_ties():
    require_gpu()
    x = np.zeros((1, 64), np.float32)
    x[0, :6] = [127.0, 0.5, 1.5, 2.5, -0.5, -2.5]
    x[0, 32:36] = [-127.0, 126.5, -3.5, 4.5]
    _check_quant(x)


def test_worked_example_a8():
    require_gpu()
    e = next(e for e in load_golden("worked_examples.json")["examples"] if e["id"] == "EX-4")
    w = {"fmt": "q4_0", "codes": (np.arange(32) % 16).astype(np.uint8)[None], "scales": np.array(e["scales"], np.uint16)}
    xq, xd, xs = quantize_gpu(np.ones((1, 32), np.float32))
    assert run_a8(w, xq, xd, xs).tolist() == e["y"]
    assert run_a8(w, xq, xd, None).tolist() == e["y"]


@pytest.mark.parametrize("n,k,m", [(1, 32, 1), (5, 64, 2), (17, 160, 4), (130, 5120, 1), (64, 5120, 4),
                                   (33, 2080, 9), (300, 512, 16)])
def test_a8_random(n, k, m):
    require_gpu()
    print(f"[a8 n={n} k={k} m={m}]", flush=True)
    g = synth.rng(n * 17 + k + m)
    w = synth.q4_0_weights(g, n, k)
    x = synth.x_f32(g, m, k)
    xq, xd, xs = quantize_gpu(x)
    rq, rd, _ = oracle.quantize_q8_0_act(x)
    ref = oracle.gemv_q4_0_a8(w, rq, rd)
    tol = oracle.gemv_q4_0_a8_abs(w, rq, rd)
    assert_within(run_a8(w, xq, xd, xs), ref, tol, f"a8 {n}x{k} m={m}")
    assert_within(run_a8(w, xq, xd, None), ref, tol, f"a8 {n}x{k} m={m} (no xs)")


def test_a8_integer_block_dots_are_exact():
    """d_w = 1 and integer x with a +-127 in every block: d_x = 1, q_x = x, and
    y is the exact integer sum of the int32 block dots."""
    require_gpu()
    g = synth.rng(21)
    n, k = 200, 5120
    w = synth.q4_0_weights(g, n, k)
    w["scales"][:] = 0x3C00
    x = g.integers(-127, 128, size=(4, k)).astype(np.float32)
    x[:, ::32] = 127.0
    xq, xd, xs = quantize_gpu(x)
    y = run_a8(w, xq, xd, xs)
    isum = oracle.block_isums_q4_0_a8(w, x.astype(np.int8))
    assert np.array_equal(y, isum.sum(axis=2).astype(np.float32))


def test_a8_batch_invariance():
    require_gpu()
    g = synth.rng(22)
    w = synth.q4_0_weights(g, 500, 5120)
    x = synth.x_f32(g, 4, 5120)
    xq, xd, xs = quantize_gpu(x)
    y4 = run_a8(w, xq, xd, xs)
    for t in range(4):
        q1, d1, s1 = quantize_gpu(x[t:t + 1])
        assert np.array_equal(run_a8(w, q1, d1, s1).view(np.uint32), y4[t:t + 1].view(np.uint32))


