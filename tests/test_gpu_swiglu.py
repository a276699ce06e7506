"""GPU parity of the fused gate+up GEMV with the SwiGLU epilogue and of the
whole dense NVFP4 MLP step (gate+up -> SwiGLU -> down), stage by stage."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.gpu_util import assert_within, dev, empty, host, pack_dev, pack_dev_gate_up, require_gpu

pytestmark = pytest.mark.gpu


def run_swiglu(w_gu, x_bits, inter):
    import torch

    k = w_gu["codes"].shape[1]
    m = x_bits.shape[0]
    a = empty((m, inter), torch.int16)
    h = empty((m, 2 * inter), torch.float32)
    qg.qgemv_nvfp4_swiglu(pack_dev_gate_up(w_gu), float(w_gu["tensor_scale"]), inter, k, dev(x_bits), m, a, h)
    return host(a).view(np.uint16), host(h)


def check_swiglu_stage(w_gu, x, inter, rows=None):
    a_bits, h = run_swiglu(w_gu, x, inter)
    sel = np.arange(inter) if rows is None else np.asarray(rows)
    both = np.concatenate([sel, sel + inter])
    assert_within(h[:, both], oracle.gemv(w_gu, x, both), oracle.gemv_abs(w_gu, x, both), "gate/up h")
    # a from the GPU's own h: within one bf16 ulp of the exact SwiGLU value
    exact = oracle.swiglu(np.concatenate([h[:, sel], h[:, sel + inter]], axis=1).astype(np.float64))
    a = oracle.decode_bf16(a_bits[:, sel])
    assert np.all(np.abs(a - exact) <= oracle.bf16_ulp(exact)), "SwiGLU output off by more than 1 bf16 ulp"
    # and it is exactly what rounding the fp64 value once gives, except where
    # the fp32 evaluation sits within rounding noise of a bf16 tie
    rne = oracle.round_to_bf16(exact)
    assert np.mean(a == rne) > 0.99
    return a_bits, h


@pytest.mark.parametrize("inter,k,m", [(16, 32, 1), (48, 64, 3), (300, 2048, 2), (512, 4096, 1), (129, 12288, 5),
                                       (64, 512, 16)])
def test_swiglu_random(inter, k, m):
    require_gpu()
    print(f"[swiglu inter={inter} k={k} m={m}]", flush=True)
    g = synth.rng(inter + k + m)
    w = synth.nvfp4_weights(g, 2 * inter, k)
    x = synth.x_bf16(g, m, k)
    check_swiglu_stage(w, x, inter)


def test_swiglu_batch_invariance():
    require_gpu()
    g = synth.rng(55)
    w = synth.nvfp4_weights(g, 2 * 256, 4096)
    x = synth.x_bf16(g, 8, 4096)
    a8, h8 = run_swiglu(w, x, 256)
    for t in range(8):
        a1, h1 = run_swiglu(w, x[t:t + 1], 256)
        assert np.array_equal(a1, a8[t:t + 1]) and np.array_equal(h1.view(np.uint32), h8[t:t + 1].view(np.uint32))


@pytest.mark.parametrize("k", [6144, 12288])
def test_swiglu_batch1_long_rows(k):
    """The SwiGLU epilogue on the LDS-staged batch-1 kernel (full rows)."""
    require_gpu()
    print(f"[swiglu batch-1 k={k}]", flush=True)
    g = synth.rng(k + 11)
    inter = 96
    w = synth.nvfp4_weights(g, 2 * inter, k)
    x = synth.x_bf16(g, 2, k)
    a1, h1 = check_swiglu_stage(w, x[:1], inter)
    a2, h2 = run_swiglu(w, x, inter)
    assert np.array_equal(a1, a2[:1]) and np.array_equal(h1.view(np.uint32), h2[:1].view(np.uint32))


@pytest.mark.parametrize("k", [4096, 8192, 12288, 16384])
def test_swiglu_two_to_four_tokens_every_token(k):
    """The SwiGLU epilogue of the LDS-staged four-slot kernels (four- and
    eight-wave workgroups): every token of m = 2, 3, 4 against the oracle, and
    bitwise against the batch-1 call on that token."""
    require_gpu()
    print(f"[swiglu m=2..4 k={k}]", flush=True)
    g = synth.rng(k + 78)
    inter = 96
    w = synth.nvfp4_weights(g, 2 * inter, k)
    x = synth.x_bf16(g, 4, k)
    singles = [run_swiglu(w, x[t:t + 1], inter) for t in range(4)]
    for m in (2, 3, 4):
        am, hm = check_swiglu_stage(w, x[:m], inter)
        for t in range(m):
            a1, h1 = singles[t]
            assert np.array_equal(am[t:t + 1], a1), (k, m, t)
            assert np.array_equal(hm[t:t + 1].view(np.uint32), h1.view(np.uint32)), (k, m, t)
