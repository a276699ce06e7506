"""GPU parity of the FP8 (E4M3) x bf16 GEMV against the oracle: the device
decoder on all 256 codes, random shapes with partial scale tiles in both scale
modes and every token class, batch invariance, special values and the full
size."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.gpu_util import assert_within, bits_equal_f32, dev, empty, fp8_fmt, host, pack_dev, require_gpu

pytestmark = pytest.mark.gpu


def run_fp8(w, x_bits):
    import torch

    n, k = w["codes"].shape
    m = x_bits.shape[0]
    y = empty((m, n), torch.float32)
    qg.qgemv_fp8(fp8_fmt(w), pack_dev(w), n, k, dev(x_bits), m, y)
    return host(y)


def check(w, x_bits, what):
    y = run_fp8(w, x_bits)
    assert_within(y, oracle.ops.gemv(w, x_bits), oracle.ops.gemv_abs(w, x_bits), what)
    return y


@pytest.mark.parametrize("tiled", [True, False])
def test_dequant_all_codes_bit_exact(tiled):
    """Every E4M3 byte through the device decoder (qg_dequant runs the GEMV's
    conversion) equals the oracle's value rounded once to fp32, NaN included."""
    import torch

    require_gpu()
    n, k = 130, 256  # two rows of tiles, the second partial
    codes = (np.arange(n * k) % 256).astype(np.uint8).reshape(n, k)
    scales = np.array([[0.5, 3.0], [0.125, 7.0]], np.float32) if tiled else np.array([[0.25]], np.float32)
    w = {"fmt": "fp8", "tiled": tiled, "codes": codes, "scales": scales}
    out = empty((n, k), torch.float32)
    qg.qg_dequant(fp8_fmt(w), pack_dev(w), 0.0, n, k, out)
    assert bits_equal_f32(host(out), oracle.ops.dequant_fp8(w).astype(np.float32))


@pytest.mark.parametrize("n,k,m,tiled", [(1, 32, 1, True), (7, 96, 3, False), (130, 160, 1, True),
                                         (257, 1056, 4, True), (1000, 4096, 1, True), (300, 12288, 2, True),
                                         (64, 256, 16, False), (129, 5120, 16, True), (33, 1024, 5, True)])
def test_random(n, k, m, tiled):
    require_gpu()
    print(f"[fp8 n={n} k={k} m={m} tiled={tiled}]", flush=True)
    g = synth.rng(n * 31 + k + m)
    w = synth.fp8_weights(g, n, k, tiled=tiled)
    check(w, synth.x_bf16(g, m, k), f"fp8 {n}x{k} m={m} tiled={tiled}")


def test_rows_are_independent_of_the_batch():
    """Token t of a batch-m call equals the batch-1 call on token t, bitwise,
    in every token class; repeated calls are bitwise identical."""
    require_gpu()
    g = synth.rng(77)
    w = synth.fp8_weights(g, 260, 2048)
    x = synth.x_bf16(g, 16, 2048)
    full = run_fp8(w, x)
    for t in (0, 3, 15):
        assert np.array_equal(run_fp8(w, x[t:t + 1]), full[t:t + 1])
    assert np.array_equal(run_fp8(w, x[:4]), full[:4])
    assert np.array_equal(run_fp8(w, x), full)


def test_special_values():
    """A NaN code makes its row NaN; zero and negative tile scales; -0 codes."""
    require_gpu()
    g = synth.rng(5)
    n, k = 256, 256
    w = synth.fp8_weights(g, n, k)
    w["scales"] = np.array([[0.0, -2.0], [1.5, 1.0]], np.float32)
    w["codes"][3, 17] = 0x7F   # NaN
    w["codes"][200, :] = 0x80  # -0 everywhere
    x = synth.x_bf16(g, 2, k)
    y = run_fp8(w, x)
    assert np.isnan(y[:, 3]).all() and not np.isnan(np.delete(y, 3, axis=1)).any()
    assert (y[:, 200] == 0).all()
    ok = np.ones(n, bool)
    ok[3] = False
    assert_within(y[:, ok], oracle.ops.gemv(w, x)[:, ok], oracle.ops.gemv_abs(w, x)[:, ok], "fp8 special")


def test_full_size_sampled():
    """The 9B-class gate+up shape, 24576 x 4096 with block-128 scales, batch 1:
    sampled rows against the oracle."""
    require_gpu()
    print("[fp8 full 24576x4096]", flush=True)
    g = synth.rng(synth.seed_for(6))
    w = synth.fp8_weights(g, 24576, 4096)
    x = synth.x_bf16(g, 1, 4096)
    y = run_fp8(w, x)
    rows = np.concatenate([np.arange(0, 24576, 97), np.arange(24570, 24576)])
    assert_within(y[:, rows], oracle.ops.gemv(w, x, rows), oracle.ops.gemv_abs(w, x, rows), "fp8 full")
