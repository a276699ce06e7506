"""GPU parity of the fused-dequant GEMVs (NVFP4 x bf16, Q8_0 x fp32) against the
oracle: worked examples, random shapes with ragged tails, exact special cases,
batch invariance, determinism and the full-size layers."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.conftest import load_golden
from tests.gpu_util import assert_within, dev, empty, host, pack_dev, require_gpu

pytestmark = pytest.mark.gpu


def run_nvfp4(w, x_bits, stream=None):
    import torch

    n, k = w["codes"].shape
    m = x_bits.shape[0]
    y = empty((m, n), torch.float32)
    qg.qgemv_nvfp4(pack_dev(w), float(w["tensor_scale"]), n, k, dev(x_bits), m, y)
    return host(y)


def run_q8(w, x):
    import torch

    n, k = w["codes"].shape
    m = x.shape[0]
    y = empty((m, n), torch.float32)
    qg.qgemv_q8_0(pack_dev(w), n, k, dev(x), m, y)
    return host(y)


def _ex(id_):
    return next(e for e in load_golden("worked_examples.json")["examples"] if e["id"] == id_)


def _pad_k(w, x, k_to=32):
    """Zero-extend a K=16 example to K=32 (the kernels take k % 32 == 0)."""
    n, k = w["codes"].shape
    if k % 32 == 0:
        return w, x
    codes = np.zeros((n, k_to), np.uint8)
    codes[:, :k] = w["codes"]
    scales = np.zeros((n, k_to // 16), np.uint8)
    scales[:, :k // 16] = w["scales"]
    xx = np.zeros((x.shape[0], k_to), x.dtype)
    xx[:, :k] = x
    return dict(w, codes=codes, scales=scales), xx


def test_worked_examples_nvfp4():
    require_gpu()
    for id_, x in (("EX-1a", np.arange(16.0)), ("EX-1b", np.array([1.0] * 8 + [0.0] * 8))):
        e = _ex(id_)
        w = {"fmt": "nvfp4", "codes": np.array(e["codes"], np.uint8), "scales": np.array(e["scales"], np.uint8),
             "tensor_scale": np.float32(e["tensor_scale"])}
        w, xb = _pad_k(w, synth.to_bf16_bits(x[None]))
        assert run_nvfp4(w, xb).tolist() == e["y"], id_
    e = _ex("EX-6")
    w = {"fmt": "nvfp4", "codes": np.array(e["codes"], np.uint8), "scales": np.array(e["scales"], np.uint8),
         "tensor_scale": np.float32(e["tensor_scale"])}
    assert run_nvfp4(w, synth.to_bf16_bits(np.array([[1.0] * 16 + [2.0] * 16]))).tolist() == e["y"]


def test_worked_examples_q8_0():
    require_gpu()
    j = np.arange(32)
    for id_, x in (("EX-2a", j.astype(np.float32)), ("EX-2b", np.ones(32, np.float32))):
        e = _ex(id_)
        w = {"fmt": "q8_0", "codes": (j - 16).astype(np.int8)[None], "scales": np.array(e["scales"], np.uint16)}
        assert run_q8(w, x[None]).tolist() == e["y"], id_
    e = _ex("EX-7")
    codes = np.zeros((2, 64), np.int8)
    codes[0, :32], codes[0, 32:], codes[1, :32], codes[1, 32:] = 1, -2, 3, 5
    w = {"fmt": "q8_0", "codes": codes, "scales": np.array(e["scales"], np.uint16)}
    assert run_q8(w, np.array([[1.0] * 32 + [-1.0] * 32], np.float32)).tolist() == e["y"]


SHAPES = [(1, 32, 1), (3, 64, 2), (17, 96, 3), (64, 512, 1), (65, 544, 4), (257, 2048, 5),
          (100, 2080, 7), (33, 4096, 9), (16, 12288, 16), (1000, 1024, 8)]


@pytest.mark.parametrize("n,k,m", SHAPES)
def test_nvfp4_random(n, k, m):
    require_gpu()
    print(f"[nvfp4 n={n} k={k} m={m}]", flush=True)
    g = synth.rng(n * 131 + k * 7 + m)
    w = synth.nvfp4_weights(g, n, k)
    x = synth.x_bf16(g, m, k)
    got = run_nvfp4(w, x)
    assert_within(got, oracle.gemv(w, x), oracle.gemv_abs(w, x), f"nvfp4 {n}x{k} m={m}")


@pytest.mark.parametrize("n,k,m", SHAPES)
def test_q8_0_random(n, k, m):
    require_gpu()
    print(f"[q8_0 n={n} k={k} m={m}]", flush=True)
    g = synth.rng(n * 131 + k * 7 + m + 5)
    w = synth.q8_0_weights(g, n, k)
    x = synth.x_f32(g, m, k)
    got = run_q8(w, x)
    assert_within(got, oracle.gemv(w, x), oracle.gemv_abs(w, x), f"q8_0 {n}x{k} m={m}")


def test_one_hot_x_is_exact():
    require_gpu()
    g = synth.rng(3)
    w = synth.nvfp4_weights(g, 50, 256)
    wq = synth.q8_0_weights(g, 50, 256)
    for col in (0, 31, 32, 255):
        x = np.zeros((1, 256), np.float32)
        x[0, col] = 1.0
        y = run_nvfp4(w, synth.to_bf16_bits(x))
        ref = oracle.dequant_nvfp4_f32(w)[:, col]  # s_t applied to the row sum: one rounding
        assert np.array_equal(y[0], ref)
        assert np.array_equal(run_q8(wq, x)[0], oracle.ops.dequant_q8_0(wq)[:, col].astype(np.float32))


def test_unit_scales_integer_x_is_exact():
    require_gpu()
    g = synth.rng(4)
    n, k = 40, 4096
    w = synth.nvfp4_weights(g, n, k, tensor_scale=1.0)
    w["scales"][:] = 0x38  # 1.0
    x = g.integers(-8, 9, size=(3, k)).astype(np.float32)
    y = run_nvfp4(w, synth.to_bf16_bits(x))
    ref = oracle.gemv(w, x)  # an exact multiple of 0.5 below 2^23
    assert np.array_equal(y, ref.astype(np.float32))
    wq = synth.q8_0_weights(g, n, k)
    wq["scales"][:] = 0x3C00
    assert np.array_equal(run_q8(wq, x), oracle.gemv(wq, x).astype(np.float32))


def test_zero_x_gives_zero():
    require_gpu()
    g = synth.rng(5)
    w = synth.nvfp4_weights(g, 20, 128)
    assert np.all(run_nvfp4(w, np.zeros((2, 128), np.uint16)) == 0)


def test_batch_invariance_and_determinism():
    require_gpu()
    g = synth.rng(6)
    for n, k in ((300, 4096), (64, 12288), (50, 512)):
        w = synth.nvfp4_weights(g, n, k)
        x = synth.x_bf16(g, 16, k)
        y16 = run_nvfp4(w, x)
        for m in (1, 2, 3, 5, 9):
            ym = run_nvfp4(w, x[:m])
            assert np.array_equal(ym.view(np.uint32), y16[:m].view(np.uint32)), (n, k, m)
        for t in range(16):
            assert np.array_equal(run_nvfp4(w, x[t:t + 1]).view(np.uint32), y16[t:t + 1].view(np.uint32))
        wq = synth.q8_0_weights(g, n, k)
        xf = synth.x_f32(g, 16, k)
        yq = run_q8(wq, xf)
        assert np.array_equal(run_q8(wq, xf[3:4]).view(np.uint32), yq[3:4].view(np.uint32))


def test_repeated_calls_are_bitwise_identical():
    import torch

    require_gpu()
    g = synth.rng(7)
    n, k = 4096, 4096
    w = synth.nvfp4_weights(g, n, k)
    x = dev(synth.x_bf16(g, 1, k))
    wd = pack_dev(w)
    ys = [empty((1, n), torch.float32) for _ in range(30)]
    for y in ys:
        qg.qgemv_nvfp4(wd, 0.01, n, k, x, 1, y)
    first = host(ys[0]).view(np.uint32)
    for y in ys[1:]:
        assert np.array_equal(host(y).view(np.uint32), first)


def test_q8_0_full_size_layer():
    """Q8_0 1024 x 1024, batch 1, every output checked."""
    require_gpu()
    case = synth.q8_gemv_case()
    got = run_q8(case.w, case.x)
    assert_within(got, oracle.gemv(case.w, case.x), oracle.gemv_abs(case.w, case.x), "q8_0 1024x1024")


@pytest.mark.parametrize("k", [6144, 8192, 12288, 16384, 5120, 7168, 10240])
def test_nvfp4_batch1_long_rows(k):
    """Batch-1 rows of three or more chunks per lane: the full ones (k a
    multiple of 2048) stage the activations in LDS, the ragged ones load them
    per lane.  Both against the oracle, and bitwise against the batch-2
    kernel (same per-row order)."""
    require_gpu()
    print(f"[nvfp4 batch-1 k={k}]", flush=True)
    g = synth.rng(k + 5)
    n = 333
    w = synth.nvfp4_weights(g, n, k)
    x = synth.x_bf16(g, 2, k)
    y1 = run_nvfp4(w, x[:1])
    assert_within(y1, oracle.gemv(w, x[:1]), oracle.gemv_abs(w, x[:1]), f"nvfp4 {n}x{k} m=1")
    y2 = run_nvfp4(w, x)
    assert np.array_equal(y1.view(np.uint32), y2[:1].view(np.uint32)), k


@pytest.mark.parametrize("k", [4096, 8192, 12288, 16384])
def test_nvfp4_two_to_four_tokens_every_token(k):
    """2-4 tokens over full rows: the four-slot kernels that stage the
    activations in LDS (four-wave workgroups at 2 and 4 chunks per lane,
    eight-wave ones at 6 and 8).  Every token of m = 2, 3, 4 against the
    oracle, and bitwise against the batch-1 call on that token."""
    require_gpu()
    print(f"[nvfp4 m=2..4 k={k}]", flush=True)
    g = synth.rng(k + 77)
    n = 333
    w = synth.nvfp4_weights(g, n, k)
    x = synth.x_bf16(g, 4, k)
    singles = [run_nvfp4(w, x[t:t + 1]) for t in range(4)]
    for m in (2, 3, 4):
        ym = run_nvfp4(w, x[:m])
        assert_within(ym, oracle.gemv(w, x[:m]), oracle.gemv_abs(w, x[:m]), f"nvfp4 {n}x{k} m={m}")
        for t in range(m):
            assert np.array_equal(ym[t:t + 1].view(np.uint32), singles[t].view(np.uint32)), (k, m, t)
