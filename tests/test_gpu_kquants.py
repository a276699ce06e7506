"""GPU parity of the K-quant (Q4_K, Q5_K, Q6_K) and IQ4_XS GEMVs with Q8_0
activations against the oracle: the verification dequantizer bit for bit,
the GEMV within the fp32 tolerance over shapes that span the launch
variants (16- and 64-lane groups, every compile-time chunk count, the
runtime-loop fallback, 1 to 16 tokens, ragged rows), extreme codes and
scales, batch invariance, and the 27B-class projection at full size."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.gpu_util import KQ_FMT, assert_within, bits_equal_f32, empty, host, pack_dev, require_gpu
from tests.test_gpu_a8 import quantize_gpu

pytestmark = pytest.mark.gpu


def run_kq(w, xq, xd, xs):
    import torch

    n, k = w["codes"].shape
    m = xq.shape[0]
    y = empty((m, n), torch.float32)
    qg.qgemv_kquant_a8(KQ_FMT[w["fmt"]], pack_dev(w), n, k, xq, xd, xs, m, y)
    return host(y)


def check(w, x, what):
    xq, xd, xs = quantize_gpu(x)
    rq, rd, _ = oracle.quantize_q8_0_act(x)
    got = run_kq(w, xq, xd, xs)
    return assert_within(got, oracle.gemv_a8(w, rq, rd), oracle.gemv_a8_abs(w, rq, rd), what)


@pytest.mark.parametrize("fmt", synth.KQUANTS)
def test_dequant_bit_exact(fmt):
    import torch

    require_gpu()
    n, k = 37, 768
    w = synth.kquant_weights(synth.rng(31), fmt, n, k)
    out = empty((n, k), torch.float32)
    qg.qg_dequant(KQ_FMT[fmt], pack_dev(w), 1.0, n, k, out)
    want = oracle.ops.dequant(w).astype(np.float32)
    # bit for bit, except that a zero compares by value: the device forms
    # sc * (q - 32) and (ls - 32) * T[q] in integers, so a product with a
    # negative factor and a zero one is +0 where the fp64 oracle gives -0
    assert bits_equal_f32(host(out), want)
    nz = want != 0
    assert np.array_equal(host(out).view(np.uint32)[nz], want.view(np.uint32)[nz])


@pytest.mark.parametrize("fmt", synth.KQUANTS)
@pytest.mark.parametrize("n,k,m", [(1, 256, 1), (5, 512, 2), (17, 768, 4), (130, 5120, 1), (64, 5120, 4),
                                   (33, 2048, 9), (300, 512, 16), (3, 16384, 5), (5, 20480, 1), (70, 1536, 3)])
def test_random(fmt, n, k, m):
    require_gpu()
    print(f"[{fmt} n={n} k={k} m={m}]", flush=True)
    g = synth.rng(n * 17 + k + m)
    w = synth.kquant_weights(g, fmt, n, k)
    check(w, synth.x_f32(g, m, k), f"{fmt} {n}x{k} m={m}")


@pytest.mark.parametrize("fmt", synth.KQUANTS)
def test_extreme_codes_and_scales(fmt):
    """Largest codes and scales, the most negative Q6_K scale, IQ4_XS scales
    0 and 63, zero super-block scales, full-range activations."""
    require_gpu()
    g = synth.rng(41)
    n, k = 64, 1024
    w = synth.kquant_weights(g, fmt, n, k)
    top = {synth.Q4_K: 15, synth.Q5_K: 31, synth.Q6_K: 63, synth.IQ4_XS: 15}[fmt]
    w["codes"][0] = top
    w["codes"][1] = 0
    if fmt == synth.Q6_K:
        w["sub"][0:2] = -128
        w["sub"][2] = 127
    else:
        w["sub"][0:2] = 63
        w["sub"][2] = 0
    if "mins" in w:
        w["mins"][0:3] = 63
    w["d"][3] = 0          # a zero super-block scale
    w["d"][4] = 0x7BFF     # the largest fp16
    x = synth.x_f32(g, 3, k)
    x[0, ::32] = 1e4       # each block's maximum maps to +127
    x[1] = -1.0            # constant blocks: every code -127
    check(w, x, f"{fmt} extreme")


@pytest.mark.parametrize("fmt", synth.KQUANTS)
def test_batch_invariance(fmt):
    require_gpu()
    g = synth.rng(42)
    w = synth.kquant_weights(g, fmt, 500, 5120)
    x = synth.x_f32(g, 4, 5120)
    xq, xd, xs = quantize_gpu(x)
    y4 = run_kq(w, xq, xd, xs)
    for t in range(4):
        q1, d1, s1 = quantize_gpu(x[t:t + 1])
        assert np.array_equal(run_kq(w, q1, d1, s1).view(np.uint32), y4[t:t + 1].view(np.uint32))


@pytest.mark.parametrize("fmt", synth.KQUANTS)
@pytest.mark.parametrize("m", [1, 4])
def test_full_size_sampled(fmt, m):
    """27B-class projection [17408 x 5120] at batch 1 and 4, sampled rows."""
    require_gpu()
    print(f"[{fmt} full m={m}]", flush=True)
    case = synth.kquant_case(fmt, m=m)
    xq, xd, xs = quantize_gpu(case.x)
    got = run_kq(case.w, xq, xd, xs)
    rq, rd, _ = oracle.quantize_q8_0_act(case.x)
    n = case.w["codes"].shape[0]
    rows = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n), synth.rng(2).integers(0, n, 240)]))
    assert_within(got[:, rows], oracle.gemv_a8(case.w, rq, rd, rows), oracle.gemv_a8_abs(case.w, rq, rd, rows),
                  f"{fmt} full m={m}")
