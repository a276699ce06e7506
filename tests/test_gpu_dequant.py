"""GPU: the device decoders are bit-exact over every (code, scale) pair."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.gpu_util import bits_equal_f32, empty, host, pack_dev, require_gpu

pytestmark = pytest.mark.gpu


def _dequant_gpu(w, s_t=1.0):
    import torch

    n, k = w["codes"].shape
    fmt = {"nvfp4": qg.QG_NVFP4, "q4_0": qg.QG_Q4_0, "q8_0": qg.QG_Q8_0}[w["fmt"]]
    out = empty((n, k), torch.float32)
    qg.qg_dequant(fmt, pack_dev(w), s_t, n, k, out)
    return host(out)


@pytest.mark.parametrize("s_t", [1.0, 0.01, 3.0e-5])
def test_nvfp4_every_code_and_scale(s_t):
    require_gpu()
    print(f"[nvfp4 dequant s_t={s_t}]", flush=True)
    codes = np.tile(np.arange(16, dtype=np.uint8), (256, 2))             # [256, 32]
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 2, 1)     # row r uses scale byte r
    w = {"fmt": "nvfp4", "codes": codes, "scales": scales, "tensor_scale": np.float32(s_t)}
    got = _dequant_gpu(w, s_t)
    ref = oracle.dequant_nvfp4_f32(w)
    assert bits_equal_f32(got, ref)


def test_q4_0_every_code_and_scale():
    require_gpu()
    print("[q4_0 dequant all scales]", flush=True)
    codes = np.tile(np.arange(16, dtype=np.uint8), (65536, 2))
    scales = np.arange(65536, dtype=np.uint32).astype(np.uint16)[:, None]
    w = {"fmt": "q4_0", "codes": codes, "scales": scales}
    got = _dequant_gpu(w)
    ref = oracle.ops.dequant_q4_0(w).astype(np.float32)
    assert bits_equal_f32(got, ref)


def test_q8_0_every_code_and_scale():
    require_gpu()
    print("[q8_0 dequant all scales]", flush=True)
    codes = np.tile(np.arange(-128, 128, dtype=np.int16).astype(np.int8), (65536, 1))  # [65536, 256]
    scales = np.repeat(np.arange(65536, dtype=np.uint32).astype(np.uint16)[:, None], 8, 1)
    w = {"fmt": "q8_0", "codes": codes, "scales": scales}
    got = _dequant_gpu(w)
    ref = oracle.ops.dequant_q8_0(w).astype(np.float32)
    assert bits_equal_f32(got, ref)


@pytest.mark.parametrize("fmt", ["nvfp4", "q4_0", "q8_0"])
def test_random_matrices(fmt):
    require_gpu()
    g = synth.rng(77)
    w = {"nvfp4": synth.nvfp4_weights, "q4_0": synth.q4_0_weights, "q8_0": synth.q8_0_weights}[fmt](g, 37, 4096)
    got = _dequant_gpu(w, 0.01)
    ref = oracle.dequant_nvfp4_f32(w) if fmt == "nvfp4" else oracle.ops.dequant(w).astype(np.float32)
    assert bits_equal_f32(got, ref)
