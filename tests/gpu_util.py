"""Helpers for the GPU parity tests: device buffers, packing, comparisons."""
from __future__ import annotations

import numpy as np
import pytest

import moe_expert_gemv_amd as qg


def require_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()  # fails loudly when the library is not built


def dev_u8(a: np.ndarray):
    """Host bytes -> device uint8 tensor (256-byte aligned)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).cuda()
    assert t.data_ptr() % 256 == 0
    return t


def dev(a: np.ndarray):
    """Host array -> device tensor of the matching dtype (uint16 travels as int16)."""
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a.copy()).cuda()
    assert t.data_ptr() % 256 == 0
    return t


def host(t, dtype=None) -> np.ndarray:
    import torch

    torch.cuda.synchronize()
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def empty(shape, dtype):
    import torch

    return torch.empty(shape, dtype=dtype, device="cuda")


KQ_FMT = {"q4_k": qg.QG_Q4_K, "q5_k": qg.QG_Q5_K, "q6_k": qg.QG_Q6_K, "iq4_xs": qg.QG_IQ4_XS}


def fp8_fmt(w: dict) -> int:
    return qg.QG_FP8_B128 if w["tiled"] else qg.QG_FP8_TENSOR


def pack_dev(w: dict):
    """Pack a logical weight dict with the library's packer and upload it."""
    if w["fmt"] == "nvfp4":
        buf = qg.qg_pack_nvfp4(w["codes"], w["scales"])
    elif w["fmt"] == "q4_0":
        buf = qg.qg_pack_q4_0(w["codes"], w["scales"])
    elif w["fmt"] == "fp8":
        buf = qg.qg_pack_fp8(fp8_fmt(w), w["codes"], w["scales"])
    elif w["fmt"] in KQ_FMT:
        buf = qg.qg_pack_kquant(KQ_FMT[w["fmt"]], w["codes"], w["d"], w["sub"], w.get("dmin"), w.get("mins"))
    else:
        buf = qg.qg_pack_q8_0(w["codes"], w["scales"])
    return dev_u8(buf)


def pack_dev_gate_up(w: dict):
    """Pack a fused gate/up NVFP4 matrix (gate rows first) with rows interleaved."""
    return dev_u8(qg.qg_pack_nvfp4_gate_up(w["codes"], w["scales"]))


def assert_within(y_gpu, y_ref, abs_sum, what=""):
    """|y_gpu - y_ref| <= 1e-5 * sum|w*x| + 1e-6 element by element."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    tol = 1e-5 * abs_sum + 1e-6
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / tol, 0)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {y_gpu[i]!r} ref {y_ref[i]!r} err {err[i]:.3e} tol {tol[i]:.3e}")
    return float(np.max(err / tol)) if err.size else 0.0


def bits_equal_f32(a, b) -> bool:
    """fp32 equality by value with NaN == NaN and +0 == -0."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and np.array_equal(a[~na], b[~nb]))
