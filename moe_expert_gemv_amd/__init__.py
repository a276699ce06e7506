"""Python binding of ``libqgemv.so``, the block-quantized GEMV library for
MI355X (gfx950).

Argument marshalling only: every function here forwards to the C entry point
of the same name declared in ``include/qgemv.h``; all arithmetic of the path
runs in the library's HIP kernels (the packers run in its C++ host code).
Device buffers are torch tensors on the current HIP device (torch provides
device memory and streams, nothing else); host buffers are numpy arrays.

If the library has not been built, every call raises ``QGLibraryMissing``
(build it with ``python -m moe_expert_gemv_amd.build``): there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "QGError", "QGLibraryMissing", "LIB_PATH", "lib", "loaded",
    "QG_NVFP4", "QG_Q8_0", "QG_Q4_0", "QG_FP8_TENSOR", "QG_FP8_B128", "QG_MAX_M", "QG_MOE_KEEP_H",
    "QG_Q4_K", "QG_Q5_K", "QG_Q6_K", "QG_IQ4_XS", "KQUANT_FORMATS", "qg_pack_kquant", "qg_unpack_kquant",
    "qgemv_kquant_a8", "qgemm_prefill_a8",
    "qg_abi_version", "qg_layout_version", "qg_status_string", "qg_packed_bytes", "qg_packed_check",
    "QG_EVERSION", "QG_NVFP4_GATE_UP", "QG_LAYOUT_VERSION",
    "qg_scale_plane_offset", "qg_pack_nvfp4", "qg_pack_nvfp4_gate_up", "qg_pack_q4_0", "qg_pack_q8_0",
    "qg_unpack_nvfp4", "qg_unpack_nvfp4_gate_up", "qg_unpack_q4_0", "qg_unpack_q8_0", "qg_pack_fp8",
    "qg_unpack_fp8", "qgemv_fp8", "fp8_scale_shape", "qg_dequant",
    "qgemv_q8_0", "qgemv_nvfp4", "qgemv_nvfp4_swiglu", "qg_quantize_q8_0_act",
    "qgemv_q4_0_a8", "moe_route_topk", "QgMoeDesc", "moe_workspace_bytes",
    "moe_gemv_grouped", "moe_forward", "moe_forward_noalloc", "QG_MOE_NOALLOC_SCRATCH_BYTES", "moe_prefill_workspace_bytes", "moe_prefill", "qgemm_prefill",
    "qgemm_prefill_workspace_bytes", "qgemm_prefill_ws", "qg_probe_read", "qg_probe_mfma_bf16",
    "QG_KERNEL_TUNED", "QG_KERNEL_GENERIC", "qg_set_kernel_policy", "qg_kernel_policy",
    "EXPORTED_SYMBOLS",
]

# QG_LIBRARY: another build of the same library to load instead (machine
# configuration, e.g. the host-sanitizer build of ``build.py --sanitize``).
LIB_PATH = os.environ.get("QG_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemv.so")

QG_OK, QG_EINVAL, QG_EUNSUPPORTED, QG_EVERSION, QG_ENOSPC, QG_EHIP = 0, -1, -2, -3, -4, -5
QG_NVFP4, QG_Q8_0, QG_Q4_0, QG_FP8_TENSOR, QG_FP8_B128 = 1, 2, 3, 4, 5
QG_Q4_K, QG_Q5_K, QG_Q6_K, QG_IQ4_XS = 6, 7, 8, 9
QG_NVFP4_GATE_UP = 10  # qg_packed_check only
QG_LAYOUT_VERSION = 2
KQUANT_FORMATS = (QG_Q4_K, QG_Q5_K, QG_Q6_K, QG_IQ4_XS)
QG_MAX_M = 16
QG_MOE_KEEP_H = 1
QG_MOE_NOALLOC_SCRATCH_BYTES = 4 << 20
QG_KERNEL_TUNED, QG_KERNEL_GENERIC = 0, 1


class QGLibraryMissing(RuntimeError):
    pass


class QGError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        text = lib().qg_status_string(status).decode()
        extra = ""
        if status == QG_EHIP:
            extra = f" (hipError {lib().qg_last_hip_error()})"
        super().__init__(f"{func}: status {status}: {text}{extra}")


class QgMoeDesc(ctypes.Structure):
    _fields_ = [
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("has_shared", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("hidden", ctypes.c_int64),
        ("inter", ctypes.c_int64),
        ("gate_up", ctypes.c_void_p),
        ("gate_up_stride", ctypes.c_int64),
        ("down", ctypes.c_void_p),
        ("down_stride", ctypes.c_int64),
        ("gate_up_scale", ctypes.c_void_p),
        ("down_scale", ctypes.c_void_p),
        ("layout_version", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]

    def __init__(self, **kw):
        kw.setdefault("layout_version", QG_LAYOUT_VERSION)
        super().__init__(**kw)


_P, _I64, _I32, _F32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

# name -> (restype, argtypes); the full exported C ABI
_SIGNATURES = {
    "qg_abi_version": (_I32, []),
    "qg_layout_version": (_I32, []),
    "qg_status_string": (ctypes.c_char_p, [_I32]),
    "qg_last_hip_error": (_I32, []),
    "qg_packed_bytes": (_SZ, [_I32, _I64, _I64]),
    "qg_packed_check": (_I32, [_I32, _P, _SZ, _I64, _I64]),
    "qg_scale_plane_offset": (_SZ, [_I32, _I64, _I64]),
    "qg_pack_nvfp4": (_I32, [_P, _P, _I64, _I64, _P, _SZ]),
    "qg_pack_nvfp4_gate_up": (_I32, [_P, _P, _I64, _I64, _P, _SZ]),
    "qg_pack_q4_0": (_I32, [_P, _P, _I64, _I64, _P, _SZ]),
    "qg_pack_q8_0": (_I32, [_P, _P, _I64, _I64, _P, _SZ]),
    "qg_unpack_nvfp4": (_I32, [_P, _SZ, _I64, _I64, _P, _P]),
    "qg_unpack_nvfp4_gate_up": (_I32, [_P, _SZ, _I64, _I64, _P, _P]),
    "qg_unpack_q4_0": (_I32, [_P, _SZ, _I64, _I64, _P, _P]),
    "qg_unpack_q8_0": (_I32, [_P, _SZ, _I64, _I64, _P, _P]),
    "qg_pack_fp8": (_I32, [_I32, _P, _P, _I64, _I64, _P, _SZ]),
    "qg_unpack_fp8": (_I32, [_I32, _P, _SZ, _I64, _I64, _P, _P]),
    "qgemv_fp8": (_I32, [_I32, _P, _I64, _I64, _P, _I64, _P, _P]),
    "qg_dequant": (_I32, [_I32, _P, _F32, _I64, _I64, _P, _P]),
    "qgemv_q8_0": (_I32, [_P, _I64, _I64, _P, _I64, _P, _P]),
    "qgemv_nvfp4": (_I32, [_P, _F32, _I64, _I64, _P, _I64, _P, _P]),
    "qgemv_nvfp4_swiglu": (_I32, [_P, _F32, _I64, _I64, _P, _I64, _P, _P, _P]),
    "qg_quantize_q8_0_act": (_I32, [_P, _I64, _I64, _P, _P, _P, _P]),
    "qgemv_q4_0_a8": (_I32, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P]),
    "qg_pack_kquant": (_I32, [_I32, _P, _P, _P, _P, _P, _I64, _I64, _P, _SZ]),
    "qg_unpack_kquant": (_I32, [_I32, _P, _SZ, _I64, _I64, _P, _P, _P, _P, _P]),
    "qgemv_kquant_a8": (_I32, [_I32, _P, _I64, _I64, _P, _P, _P, _I64, _P, _P]),
    "qgemm_prefill_a8": (_I32, [_P, _I64, _I64, _P, _P, _I64, _P, _P]),
    "moe_route_topk": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "moe_workspace_bytes": (_SZ, [ctypes.POINTER(QgMoeDesc), _I64]),
    "moe_gemv_grouped": (_I32, [ctypes.POINTER(QgMoeDesc), _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "moe_forward": (_I32, [ctypes.POINTER(QgMoeDesc), _P, _P, _I64, _P, _P, _SZ, _P]),
    "moe_forward_noalloc": (_I32, [ctypes.POINTER(QgMoeDesc), _P, _P, _I64, _P, _P]),
    "moe_prefill_workspace_bytes": (_SZ, [ctypes.POINTER(QgMoeDesc), _I64]),
    "moe_prefill": (_I32, [ctypes.POINTER(QgMoeDesc), _P, _P, _I64, _P, _P, _SZ, _P]),
    "qgemm_prefill": (_I32, [_P, _F32, _I64, _I64, _P, _I64, _P, _P]),
    "qgemm_prefill_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "qgemm_prefill_ws": (_I32, [_P, _F32, _I64, _I64, _P, _I64, _P, _P, _SZ, _P]),
    "qg_probe_read": (_I32, [_P, _SZ, _I32, _P, _P]),
    "qg_probe_mfma_bf16": (_I32, [_I64, _P, ctypes.POINTER(ctypes.c_int64), _P]),
    "qg_set_kernel_policy": (_I32, [_I32]),
    "qg_kernel_policy": (_I32, []),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QGLibraryMissing(
                f"{LIB_PATH} is not built; run `python -m moe_expert_gemv_amd.build` first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def loaded() -> bool:
    return _lib is not None


def _check(func: str, status: int) -> None:
    if status != QG_OK:
        raise QGError(func, status)


# ---------------------------------------------------------------- marshalling

def _dptr(t):
    """Device pointer of a torch tensor (or None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _hptr(a: np.ndarray):
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("expected a C-contiguous array")
    return a.ctypes.data


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ---------------------------------------------------------------- versions / sizes

def qg_abi_version() -> int:
    return lib().qg_abi_version()


def qg_layout_version() -> int:
    return lib().qg_layout_version()


def qg_status_string(status: int) -> str:
    return lib().qg_status_string(status).decode()


def qg_packed_bytes(fmt: int, n: int, k: int) -> int:
    return lib().qg_packed_bytes(fmt, n, k)


def qg_packed_check(fmt: int, buf, n: int, k: int) -> int:
    """Status of a packed host buffer's stamp against (fmt, n, k): QG_OK,
    QG_EVERSION, QG_EINVAL or QG_ENOSPC (returned, not raised)."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    return int(lib().qg_packed_check(fmt, _hptr(buf), buf.nbytes, n, k))


def qg_scale_plane_offset(fmt: int, n: int, k: int) -> int:
    return lib().qg_scale_plane_offset(fmt, n, k)


# ---------------------------------------------------------------- packers (host)

def _pack(func, fmt, codes, scales, code_dtype, scale_dtype):
    codes = np.ascontiguousarray(codes, dtype=code_dtype)
    scales = np.ascontiguousarray(scales, dtype=scale_dtype)
    n, k = codes.shape
    size = qg_packed_bytes(fmt, n, k)
    if size == 0:
        raise QGError(func, QG_EINVAL)
    out = np.empty(size, dtype=np.uint8)
    _check(func, getattr(lib(), func)(_hptr(codes), _hptr(scales), n, k, _hptr(out), size))
    return out


def qg_pack_nvfp4(codes, scales_e4m3) -> np.ndarray:
    return _pack("qg_pack_nvfp4", QG_NVFP4, codes, scales_e4m3, np.uint8, np.uint8)


def qg_pack_nvfp4_gate_up(codes, scales_e4m3) -> np.ndarray:
    """Fused gate/up matrix [2*inter][k] (gate rows first) -> packed, rows interleaved."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales_e4m3, dtype=np.uint8)
    n, k = codes.shape
    if n % 2:
        raise QGError("qg_pack_nvfp4_gate_up", QG_EINVAL)
    size = qg_packed_bytes(QG_NVFP4, n, k)
    if size == 0:
        raise QGError("qg_pack_nvfp4_gate_up", QG_EINVAL)
    out = np.empty(size, dtype=np.uint8)
    _check("qg_pack_nvfp4_gate_up",
           lib().qg_pack_nvfp4_gate_up(_hptr(codes), _hptr(scales), n // 2, k, _hptr(out), size))
    return out


def qg_pack_q4_0(codes, scales_f16) -> np.ndarray:
    return _pack("qg_pack_q4_0", QG_Q4_0, codes, scales_f16, np.uint8, np.uint16)


def qg_pack_q8_0(codes, scales_f16) -> np.ndarray:
    return _pack("qg_pack_q8_0", QG_Q8_0, codes, scales_f16, np.int8, np.uint16)


def _unpack(func, buf, n, k, code_dtype, scale_dtype, blk):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    codes = np.empty((n, k), dtype=code_dtype)
    scales = np.empty((n, k // blk), dtype=scale_dtype)
    _check(func, getattr(lib(), func)(_hptr(buf), buf.nbytes, n, k, _hptr(codes), _hptr(scales)))
    return codes, scales


def qg_unpack_nvfp4(buf, n, k):
    return _unpack("qg_unpack_nvfp4", buf, n, k, np.uint8, np.uint8, 16)


def qg_unpack_nvfp4_gate_up(buf, inter, k):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    codes = np.empty((2 * inter, k), dtype=np.uint8)
    scales = np.empty((2 * inter, k // 16), dtype=np.uint8)
    _check("qg_unpack_nvfp4_gate_up",
           lib().qg_unpack_nvfp4_gate_up(_hptr(buf), buf.nbytes, inter, k, _hptr(codes), _hptr(scales)))
    return codes, scales


def qg_unpack_q4_0(buf, n, k):
    return _unpack("qg_unpack_q4_0", buf, n, k, np.uint8, np.uint16, 32)


def qg_unpack_q8_0(buf, n, k):
    return _unpack("qg_unpack_q8_0", buf, n, k, np.int8, np.uint16, 32)


def fp8_scale_shape(fmt, n, k):
    """Shape of the fp32 scales of an FP8 matrix: (1, 1) per tensor, the
    [ceil(n/128), ceil(k/128)] tile grid for block-128."""
    if fmt == QG_FP8_TENSOR:
        return (1, 1)
    if fmt == QG_FP8_B128:
        return ((n + 127) // 128, (k + 127) // 128)
    raise QGError("fp8_scale_shape", QG_EINVAL)


def qg_pack_fp8(fmt, codes, scales) -> np.ndarray:
    """E4M3 codes [n][k] (bit patterns) and fp32 scales (fp8_scale_shape) -> packed."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = codes.shape
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    if scales.size != int(np.prod(fp8_scale_shape(fmt, n, k))):
        raise QGError("qg_pack_fp8", QG_EINVAL)
    size = qg_packed_bytes(fmt, n, k)
    if size == 0:
        raise QGError("qg_pack_fp8", QG_EINVAL)
    out = np.empty(size, dtype=np.uint8)
    _check("qg_pack_fp8", lib().qg_pack_fp8(fmt, _hptr(codes), _hptr(scales), n, k, _hptr(out), size))
    return out


def qg_unpack_fp8(fmt, buf, n, k):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    codes = np.empty((n, k), dtype=np.uint8)
    scales = np.empty(fp8_scale_shape(fmt, n, k), dtype=np.float32)
    _check("qg_unpack_fp8", lib().qg_unpack_fp8(fmt, _hptr(buf), buf.nbytes, n, k, _hptr(codes), _hptr(scales)))
    return codes, scales


def _kq_has_min(fmt):
    return fmt in (QG_Q4_K, QG_Q5_K)


def qg_pack_kquant(fmt, codes, d, sub, dmin=None, mins=None) -> np.ndarray:
    """K-quant / IQ4_XS logical arrays -> packed host buffer.  codes [n][k]
    uint8; d (and dmin) fp16 bits [n][k/256]; sub [n][k/32] (Q6_K: int8
    [n][k/16]); mins [n][k/32] (Q4_K / Q5_K)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = codes.shape
    size = qg_packed_bytes(fmt, n, k)
    if size == 0:
        raise QGError("qg_pack_kquant", QG_EINVAL)
    d = np.ascontiguousarray(d, dtype=np.uint16)
    sub = np.ascontiguousarray(sub).view(np.uint8) if np.asarray(sub).dtype == np.int8 else \
        np.ascontiguousarray(sub, dtype=np.uint8)
    want_sub = n * (k // 16 if fmt == QG_Q6_K else k // 32)
    if d.size != n * (k // 256) or sub.size != want_sub:
        raise QGError("qg_pack_kquant", QG_EINVAL)
    dm = mn = None
    if _kq_has_min(fmt):
        if dmin is None or mins is None:
            raise QGError("qg_pack_kquant", QG_EINVAL)
        dm = np.ascontiguousarray(dmin, dtype=np.uint16)
        mn = np.ascontiguousarray(mins, dtype=np.uint8)
        if dm.size != d.size or mn.size != n * (k // 32):
            raise QGError("qg_pack_kquant", QG_EINVAL)
    out = np.empty(size, dtype=np.uint8)
    _check("qg_pack_kquant", lib().qg_pack_kquant(fmt, _hptr(codes), _hptr(d), None if dm is None else _hptr(dm),
                                                  _hptr(sub), None if mn is None else _hptr(mn), n, k,
                                                  _hptr(out), size))
    return out


def qg_unpack_kquant(fmt, buf, n, k) -> dict:
    """Inverse of qg_pack_kquant: {"codes", "d", "sub"[, "dmin", "mins"]}."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    codes = np.empty((n, k), dtype=np.uint8)
    d = np.empty((n, k // 256), dtype=np.uint16)
    sub = np.empty((n, k // 16 if fmt == QG_Q6_K else k // 32), dtype=np.uint8)
    dm = np.empty_like(d) if _kq_has_min(fmt) else None
    mn = np.empty((n, k // 32), dtype=np.uint8) if _kq_has_min(fmt) else None
    _check("qg_unpack_kquant",
           lib().qg_unpack_kquant(fmt, _hptr(buf), buf.nbytes, n, k, _hptr(codes), _hptr(d),
                                  None if dm is None else _hptr(dm), _hptr(sub), None if mn is None else _hptr(mn)))
    out = {"codes": codes, "d": d, "sub": sub.view(np.int8) if fmt == QG_Q6_K else sub}
    if dm is not None:
        out["dmin"], out["mins"] = dm, mn
    return out


# ---------------------------------------------------------------- device entry points

def qg_dequant(fmt, w, tensor_scale, n, k, out, stream=None) -> None:
    _check("qg_dequant", lib().qg_dequant(fmt, _dptr(w), tensor_scale, n, k, _dptr(out), _stream(stream)))


def qgemv_q8_0(w, n, k, x, m, y, stream=None) -> None:
    _check("qgemv_q8_0", lib().qgemv_q8_0(_dptr(w), n, k, _dptr(x), m, _dptr(y), _stream(stream)))


def qgemv_nvfp4(w, tensor_scale, n, k, x, m, y, stream=None) -> None:
    _check("qgemv_nvfp4",
           lib().qgemv_nvfp4(_dptr(w), tensor_scale, n, k, _dptr(x), m, _dptr(y), _stream(stream)))


def qgemv_fp8(fmt, w, n, k, x, m, y, stream=None) -> None:
    _check("qgemv_fp8", lib().qgemv_fp8(fmt, _dptr(w), n, k, _dptr(x), m, _dptr(y), _stream(stream)))


def qgemv_nvfp4_swiglu(w_gu, tensor_scale, inter, k, x, m, a, h=None, stream=None) -> None:
    _check("qgemv_nvfp4_swiglu",
           lib().qgemv_nvfp4_swiglu(_dptr(w_gu), tensor_scale, inter, k, _dptr(x), m, _dptr(a),
                                    _dptr(h), _stream(stream)))


def qg_quantize_q8_0_act(x, m, k, xq, xd, xs=None, stream=None) -> None:
    _check("qg_quantize_q8_0_act",
           lib().qg_quantize_q8_0_act(_dptr(x), m, k, _dptr(xq), _dptr(xd), _dptr(xs), _stream(stream)))


def qgemv_q4_0_a8(w, n, k, xq, xd, xs, m, y, stream=None) -> None:
    _check("qgemv_q4_0_a8",
           lib().qgemv_q4_0_a8(_dptr(w), n, k, _dptr(xq), _dptr(xd), _dptr(xs), m, _dptr(y),
                               _stream(stream)))


def qgemv_kquant_a8(fmt, w, n, k, xq, xd, xs, m, y, stream=None) -> None:
    _check("qgemv_kquant_a8",
           lib().qgemv_kquant_a8(fmt, _dptr(w), n, k, _dptr(xq), _dptr(xd), _dptr(xs), m, _dptr(y),
                                 _stream(stream)))


def qgemm_prefill_a8(w, n, k, xq, xd, m, y, stream=None) -> None:
    _check("qgemm_prefill_a8",
           lib().qgemm_prefill_a8(_dptr(w), n, k, _dptr(xq), _dptr(xd), m, _dptr(y), _stream(stream)))


def moe_route_topk(logits, t, n_experts, top_k, ids, weights, stream=None) -> None:
    _check("moe_route_topk",
           lib().moe_route_topk(_dptr(logits), t, n_experts, top_k, _dptr(ids), _dptr(weights),
                                _stream(stream)))


def moe_workspace_bytes(desc: QgMoeDesc, t: int) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(desc), t)


def moe_gemv_grouped(desc: QgMoeDesc, x, ids, weights, t, y, ws, ws_bytes=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_gemv_grouped",
           lib().moe_gemv_grouped(ctypes.byref(desc), _dptr(x), _dptr(ids), _dptr(weights), t,
                                  _dptr(y), _dptr(ws), nbytes, _stream(stream)))


def moe_forward(desc: QgMoeDesc, x, logits, t, y, ws, ws_bytes=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_forward",
           lib().moe_forward(ctypes.byref(desc), _dptr(x), _dptr(logits), t, _dptr(y), _dptr(ws), nbytes,
                             _stream(stream)))


def moe_forward_noalloc(desc: QgMoeDesc, x, logits, t, y, stream=None) -> None:
    _check("moe_forward_noalloc",
           lib().moe_forward_noalloc(ctypes.byref(desc), _dptr(x), _dptr(logits), t, _dptr(y), _stream(stream)))


def moe_prefill_workspace_bytes(desc: QgMoeDesc, t: int) -> int:
    return lib().moe_prefill_workspace_bytes(ctypes.byref(desc), t)


def moe_prefill(desc: QgMoeDesc, x, logits, t, y, ws, ws_bytes=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_prefill",
           lib().moe_prefill(ctypes.byref(desc), _dptr(x), _dptr(logits), t, _dptr(y), _dptr(ws), nbytes,
                             _stream(stream)))


def qgemm_prefill(w, tensor_scale, n, k, x, m, y, stream=None) -> None:
    _check("qgemm_prefill",
           lib().qgemm_prefill(_dptr(w), tensor_scale, n, k, _dptr(x), m, _dptr(y), _stream(stream)))


def qgemm_prefill_workspace_bytes(n, k, m) -> int:
    return int(lib().qgemm_prefill_workspace_bytes(n, k, m))


def qgemm_prefill_ws(w, tensor_scale, n, k, x, m, y, ws, ws_bytes=None, stream=None) -> None:
    if ws is None:
        ptr, nbytes = 0, 0 if ws_bytes is None else ws_bytes
    else:
        ptr = _dptr(ws)
        nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("qgemm_prefill_ws",
           lib().qgemm_prefill_ws(_dptr(w), tensor_scale, n, k, _dptr(x), m, _dptr(y), ptr, nbytes,
                                  _stream(stream)))


def qg_probe_read(buf, wg_per_cu, sink, stream=None) -> None:
    """Stream the device tensor buf once (achievable read bandwidth probe)."""
    _check("qg_probe_read", lib().qg_probe_read(_dptr(buf), buf.numel() * buf.element_size(), wg_per_cu,
                                                _dptr(sink), _stream(stream)))


def qg_probe_mfma_bf16(iters, sink, stream=None) -> int:
    """Launch the bf16 MFMA peak probe; returns the flops it performs."""
    flops = ctypes.c_int64(0)
    _check("qg_probe_mfma_bf16", lib().qg_probe_mfma_bf16(iters, _dptr(sink), ctypes.byref(flops), _stream(stream)))
    return int(flops.value)


def qg_set_kernel_policy(policy: int) -> None:
    """Select the tuned (default) or the generic kernels for the calls that
    have both (the library's rollback seam; QG_FORCE_KERNEL sets the start)."""
    _check("qg_set_kernel_policy", lib().qg_set_kernel_policy(policy))


def qg_kernel_policy() -> int:
    return int(lib().qg_kernel_policy())
