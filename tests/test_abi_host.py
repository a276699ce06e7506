"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol the header declares, packs and unpacks exactly, and rejects bad
arguments before touching the GPU."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import moe_expert_gemv_amd as qg
import synth

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qg.LIB_PATH):
        pytest.fail("libqgemv.so is not built (python -m moe_expert_gemv_amd.build)")
    return qg.lib()


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_header_and_binding_agree():
    assert _header_functions() == sorted(qg.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", qg.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [s for s in _header_functions() if s not in exported]
    assert not missing, missing
    for s in _header_functions():
        assert hasattr(L, s)


def test_versions_and_status_strings(L):
    assert qg.qg_abi_version() == 2
    assert qg.qg_layout_version() == qg.QG_LAYOUT_VERSION == 2
    for s in (0, -1, -2, -3, -4, -5):
        assert qg.qg_status_string(s) and qg.qg_status_string(s) != "unknown status"
    assert qg.qg_status_string(12345) == "unknown status"


@pytest.mark.parametrize("fmt,n,k,codes,scales", [
    (qg.QG_NVFP4, 3, 64, 96, 12), (qg.QG_Q4_0, 3, 64, 96, 12), (qg.QG_Q8_0, 3, 64, 192, 12),
    (qg.QG_NVFP4, 24576, 4096, 50331648, 6291456),
])
def test_packed_sizes(L, fmt, n, k, codes, scales):
    off = qg.qg_scale_plane_offset(fmt, n, k)
    assert off % 256 == 0 and off >= codes and off - codes < 256
    total = qg.qg_packed_bytes(fmt, n, k) - 256  # the layout stamp closes the buffer
    assert total % 256 == 0 and total - off >= scales and total - off - scales < 256


@pytest.mark.parametrize("fmt,n,k", [(qg.QG_NVFP4, 1, 16), (qg.QG_NVFP4, 0, 32), (qg.QG_Q8_0, 4, 48),
                                     (7, 4, 32), (qg.QG_Q4_0, -1, 32)])
def test_packed_bytes_rejects_bad_shapes(L, fmt, n, k):
    assert qg.qg_packed_bytes(fmt, n, k) == 0


def _roundtrip(fmt, w):
    if fmt == qg.QG_NVFP4:
        buf = qg.qg_pack_nvfp4(w["codes"], w["scales"])
        c, s = qg.qg_unpack_nvfp4(buf, *w["codes"].shape)
    elif fmt == qg.QG_Q4_0:
        buf = qg.qg_pack_q4_0(w["codes"], w["scales"])
        c, s = qg.qg_unpack_q4_0(buf, *w["codes"].shape)
    else:
        buf = qg.qg_pack_q8_0(w["codes"], w["scales"])
        c, s = qg.qg_unpack_q8_0(buf, *w["codes"].shape)
    assert np.array_equal(c, w["codes"]) and np.array_equal(s, w["scales"])
    return buf


@pytest.mark.parametrize("n,k", [(1, 32), (3, 64), (17, 96), (64, 2048)])
def test_pack_roundtrip(L, n, k):
    g = synth.rng(n * 1000 + k)
    _roundtrip(qg.QG_NVFP4, synth.nvfp4_weights(g, n, k))
    _roundtrip(qg.QG_Q4_0, synth.q4_0_weights(g, n, k))
    _roundtrip(qg.QG_Q8_0, synth.q8_0_weights(g, n, k))


def test_pack_layout_is_as_documented(L):
    # NVFP4: byte j = element 2j (low nibble) | element 2j+1 (high nibble)
    codes = np.arange(64, dtype=np.uint8).reshape(2, 32) % 16
    scales = np.arange(4, dtype=np.uint8).reshape(2, 2) + 0x30
    buf = qg.qg_pack_nvfp4(codes, scales)
    assert buf[0] == (codes[0, 0] | codes[0, 1] << 4) and buf[16] == (codes[1, 0] | codes[1, 1] << 4)
    off = qg.qg_scale_plane_offset(qg.QG_NVFP4, 2, 32)
    assert buf[off:off + 4].tolist() == [0x30, 0x31, 0x32, 0x33]
    # Q4_0: byte i of a block = element i (low) | element 16+i (high)
    q = (np.arange(32, dtype=np.uint8) % 16)[None]
    buf = qg.qg_pack_q4_0(q, np.array([[0x3C00]], np.uint16))
    assert all(buf[i] == (q[0, i] | q[0, 16 + i] << 4) for i in range(16))
    off = qg.qg_scale_plane_offset(qg.QG_Q4_0, 1, 32)
    assert buf[off] == 0x00 and buf[off + 1] == 0x3C


def test_gate_up_pack_interleaves_rows(L):
    g = synth.rng(12)
    w = synth.nvfp4_weights(g, 2 * 5, 64)
    buf = qg.qg_pack_nvfp4_gate_up(w["codes"], w["scales"])
    c, s = qg.qg_unpack_nvfp4_gate_up(buf, 5, 64)
    assert np.array_equal(c, w["codes"]) and np.array_equal(s, w["scales"])
    # the same bytes as the plain packer applied to the interleaved row order
    order = np.ravel(np.column_stack([np.arange(5), 5 + np.arange(5)]))
    plain = qg.qg_pack_nvfp4(w["codes"][order], w["scales"][order])
    assert np.array_equal(buf[:-256], plain[:-256])  # all but the stamp, which names the row order
    assert buf[-256 + 12] == 1 and plain[-256 + 12] == 0


@settings(max_examples=40, deadline=None)
@given(n=st.integers(1, 9), kb=st.integers(1, 6), seed=st.integers(0, 2 ** 31 - 1))
def test_pack_roundtrip_property(n, kb, seed):
    qg.lib()
    g = np.random.default_rng(seed)
    k = 32 * kb
    nv = {"codes": g.integers(0, 16, (n, k), dtype=np.uint8), "scales": g.integers(0, 256, (n, k // 16), dtype=np.uint8)}
    q4 = {"codes": g.integers(0, 16, (n, k), dtype=np.uint8), "scales": g.integers(0, 65536, (n, k // 32)).astype(np.uint16)}
    q8 = {"codes": g.integers(-128, 128, (n, k), dtype=np.int8), "scales": g.integers(0, 65536, (n, k // 32)).astype(np.uint16)}
    _roundtrip(qg.QG_NVFP4, nv)
    _roundtrip(qg.QG_Q4_0, q4)
    _roundtrip(qg.QG_Q8_0, q8)


def test_pack_rejects_out_of_range_codes(L):
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 5] = 16
    with pytest.raises(qg.QGError) as e:
        qg.qg_pack_nvfp4(codes, np.zeros((1, 2), np.uint8))
    assert e.value.status == qg.QG_EINVAL
    with pytest.raises(qg.QGError):
        qg.qg_pack_q4_0(codes, np.zeros((1, 1), np.uint16))


def test_pack_rejects_small_destination(L):
    codes = np.zeros((2, 32), np.uint8)
    scales = np.zeros((2, 2), np.uint8)
    buf = np.zeros(100, np.uint8)
    st_ = L.qg_pack_nvfp4(codes.ctypes.data, scales.ctypes.data, 2, 32, buf.ctypes.data, buf.nbytes)
    assert st_ == qg.QG_ENOSPC
    assert L.qg_pack_nvfp4(None, scales.ctypes.data, 2, 32, buf.ctypes.data, 1 << 20) == qg.QG_EINVAL


# Host-side validation of the device entry points: each bad call must return
# its status before any HIP call, so these run without a GPU.  Pointers are
# fake but aligned; they are never dereferenced.
FAKE = 0x7F0000000000


def test_gemv_argument_checks(L):
    f = L.qgemv_nvfp4
    assert f(None, 1.0, 8, 64, FAKE, 1, FAKE, None) == qg.QG_EINVAL          # null weights
    assert f(FAKE + 16, 1.0, 8, 64, FAKE, 1, FAKE, None) == qg.QG_EINVAL     # misaligned weights
    assert f(FAKE, 1.0, 8, 64, FAKE + 2, 1, FAKE, None) == qg.QG_EINVAL      # misaligned x
    assert f(FAKE, 1.0, 8, 48, FAKE, 1, FAKE, None) == qg.QG_EINVAL          # k % 32 != 0
    assert f(FAKE, 1.0, 0, 64, FAKE, 1, FAKE, None) == qg.QG_EINVAL          # n = 0
    assert f(FAKE, 1.0, 8, 64, FAKE, 0, FAKE, None) == qg.QG_EINVAL          # m = 0
    assert f(FAKE, 1.0, 8, 64, FAKE, 17, FAKE, None) == qg.QG_EUNSUPPORTED   # m > 16
    assert L.qgemv_q8_0(FAKE, 8, 64, FAKE, 17, FAKE, None) == qg.QG_EUNSUPPORTED
    assert L.qgemv_q4_0_a8(FAKE, 8, 64, FAKE, None, None, 1, FAKE, None) == qg.QG_EINVAL  # null xd
    assert L.qgemv_nvfp4_swiglu(FAKE, 1.0, 0, 64, FAKE, 1, FAKE, None, None) == qg.QG_EINVAL
    assert L.qg_quantize_q8_0_act(FAKE, 1, 40, FAKE, FAKE, None, None) == qg.QG_EINVAL
    assert L.qg_dequant(9, FAKE, 1.0, 8, 64, FAKE, None) == qg.QG_EINVAL
    assert L.qgemm_prefill(FAKE, 1.0, 8, 64, FAKE, 0, FAKE, None) == qg.QG_EINVAL


def test_prefill_workspace_size_and_checks(L):
    """qgemm_prefill_ws: workspace size rule and argument errors (checked on
    the host before any launch)."""
    f = L.qgemm_prefill_ws
    need = qg.qgemm_prefill_workspace_bytes(12288, 4160, 64)
    assert need == 5 * 64 * 12288 * 4                      # ceil(k/1024) slices of fp32 [m][n]
    assert qg.qgemm_prefill_workspace_bytes(100, 1056, 7) == 2 * 7 * 100 * 4
    assert qg.qgemm_prefill_workspace_bytes(12288, 4096, 64) == 0   # k a multiple of 256: one pass
    assert qg.qgemm_prefill_workspace_bytes(300, 768, 128) == 0
    assert qg.qgemm_prefill_workspace_bytes(12288, 4096, 512) == 0  # m > 128: no workspace
    assert qg.qgemm_prefill_workspace_bytes(8, 48, 1) == 0          # invalid k
    assert qg.qgemm_prefill_workspace_bytes(8, 64, 0) == 0          # invalid m
    assert f(FAKE, 1.0, 12288, 4160, FAKE, 64, FAKE, None, need, None) == qg.QG_EINVAL       # null ws
    assert f(FAKE, 1.0, 12288, 4160, FAKE, 64, FAKE, FAKE + 16, need, None) == qg.QG_EINVAL  # misaligned ws
    assert f(FAKE, 1.0, 12288, 4160, FAKE, 64, FAKE, FAKE, need - 4, None) == qg.QG_ENOSPC   # too small
    assert f(FAKE, 1.0, 8, 64, FAKE, 0, FAKE, FAKE, 1 << 20, None) == qg.QG_EINVAL           # m = 0
    assert f(None, 1.0, 8, 64, FAKE, 1, FAKE, FAKE, 1 << 20, None) == qg.QG_EINVAL           # null w


def test_router_argument_checks(L):
    f = L.moe_route_topk
    assert f(None, 1, 256, 8, FAKE, FAKE, None) == qg.QG_EINVAL
    assert f(FAKE, 1, 4, 8, FAKE, FAKE, None) == qg.QG_EINVAL        # top_k > n_experts
    assert f(FAKE, 1, 2048, 8, FAKE, FAKE, None) == qg.QG_EUNSUPPORTED
    assert f(FAKE, 1, 256, 17, FAKE, FAKE, None) == qg.QG_EUNSUPPORTED


def _desc(**kw):
    gu = qg.qg_packed_bytes(qg.QG_NVFP4, 1024, 2048)
    dn = qg.qg_packed_bytes(qg.QG_NVFP4, 2048, 512)
    d = qg.QgMoeDesc(n_experts=256, top_k=8, has_shared=1, flags=0, hidden=2048, inter=512,
                     gate_up=FAKE, gate_up_stride=gu, down=FAKE, down_stride=dn,
                     gate_up_scale=FAKE, down_scale=FAKE)
    for key, v in kw.items():
        setattr(d, key, v)
    return d


def test_moe_workspace_and_checks(L):
    d = _desc()
    ws1 = qg.moe_workspace_bytes(d, 1)
    ws4 = qg.moe_workspace_bytes(d, 4)
    assert ws1 > 0 and ws4 > ws1 and ws1 % 256 == 0
    assert qg.moe_workspace_bytes(d, 17) == 0
    assert qg.moe_workspace_bytes(_desc(top_k=9), 1) == 0
    assert qg.moe_workspace_bytes(_desc(gate_up_stride=1024), 1) == 0
    f = L.moe_gemv_grouped
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 1, FAKE, FAKE, ws1 - 256, None) == qg.QG_ENOSPC
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 17, FAKE, FAKE, 1 << 30, None) == qg.QG_EUNSUPPORTED
    assert f(ctypes.byref(_desc(down=None)), FAKE, FAKE, FAKE, 1, FAKE, FAKE, ws1, None) == qg.QG_EINVAL
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 1, FAKE, FAKE + 16, ws1, None) == qg.QG_EINVAL


def test_moe_forward_checks(L):
    d = _desc()
    ws1 = qg.moe_workspace_bytes(d, 1)
    f = L.moe_forward
    assert f(ctypes.byref(d), FAKE, FAKE, 1, FAKE, FAKE, ws1 - 256, None) == qg.QG_ENOSPC
    assert f(ctypes.byref(d), FAKE, None, 1, FAKE, FAKE, ws1, None) == qg.QG_EINVAL
    assert f(ctypes.byref(d), FAKE, FAKE, 0, FAKE, FAKE, ws1, None) == qg.QG_EINVAL
    assert f(ctypes.byref(_desc(n_experts=2048)), FAKE, FAKE, 1, FAKE, FAKE, 1 << 30, None) == qg.QG_EUNSUPPORTED


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(qg, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(qg, "_lib", None)
    with pytest.raises(qg.QGLibraryMissing):
        qg.qg_abi_version()


# ---------------------------------------------------------------- FP8

@pytest.mark.parametrize("fmt,n,k,scales", [(qg.QG_FP8_TENSOR, 3, 64, 4), (qg.QG_FP8_B128, 3, 64, 4),
                                            (qg.QG_FP8_B128, 300, 384, 3 * 3 * 4),
                                            (qg.QG_FP8_B128, 24576, 4096, 192 * 32 * 4)])
def test_fp8_packed_sizes(L, fmt, n, k, scales):
    off = qg.qg_scale_plane_offset(fmt, n, k)
    assert off % 256 == 0 and off >= n * k and off - n * k < 256
    total = qg.qg_packed_bytes(fmt, n, k) - 256  # the layout stamp closes the buffer
    assert total % 256 == 0 and total - off >= scales and total - off - scales < 256


@pytest.mark.parametrize("n,k,tiled", [(1, 32, True), (3, 64, False), (130, 160, True), (300, 384, True)])
def test_fp8_pack_roundtrip_and_layout(L, n, k, tiled):
    g = synth.rng(n * 7 + k)
    w = synth.fp8_weights(g, n, k, tiled=tiled)
    fmt = qg.QG_FP8_B128 if tiled else qg.QG_FP8_TENSOR
    buf = qg.qg_pack_fp8(fmt, w["codes"], w["scales"])
    c, s = qg.qg_unpack_fp8(fmt, buf, n, k)
    assert np.array_equal(c, w["codes"]) and np.array_equal(s, w["scales"])
    # codes plane: row-major bytes; scale plane: the fp32 grid, row-major
    assert np.array_equal(buf[:n * k].reshape(n, k), w["codes"])
    off = qg.qg_scale_plane_offset(fmt, n, k)
    assert np.array_equal(buf[off:off + 4 * w["scales"].size].view(np.float32).reshape(w["scales"].shape),
                          w["scales"])


def test_fp8_argument_checks(L):
    codes = np.zeros((4, 64), np.uint8)
    with pytest.raises(qg.QGError):
        qg.qg_pack_fp8(qg.QG_NVFP4, codes, np.ones((1, 1), np.float32))  # not an FP8 format
    with pytest.raises(qg.QGError):
        qg.qg_pack_fp8(qg.QG_FP8_B128, codes, np.ones((2, 2), np.float32))  # wrong grid size
    assert L.qgemv_fp8(qg.QG_NVFP4, 256, 4, 64, 256, 1, 256, None) == qg.QG_EINVAL  # bad format
    assert L.qgemv_fp8(qg.QG_FP8_B128, 256, 4, 48, 256, 1, 256, None) == qg.QG_EINVAL  # k % 32
    assert L.qgemv_fp8(qg.QG_FP8_B128, 256, 4, 64, 256, 17, 256, None) == qg.QG_EUNSUPPORTED  # m > 16
    assert L.qgemv_fp8(qg.QG_FP8_TENSOR, 0, 4, 64, 256, 1, 256, None) == qg.QG_EINVAL  # null w


# ---------------------------------------------------------------- K-quants

KQ = {synth.Q4_K: qg.QG_Q4_K, synth.Q5_K: qg.QG_Q5_K, synth.Q6_K: qg.QG_Q6_K, synth.IQ4_XS: qg.QG_IQ4_XS}


def _kq_pack(w):
    return qg.qg_pack_kquant(KQ[w["fmt"]], w["codes"], w["d"], w["sub"], w.get("dmin"), w.get("mins"))


@pytest.mark.parametrize("fmt", synth.KQUANTS)
@pytest.mark.parametrize("n,k", [(1, 256), (7, 768), (33, 5120)])
def test_kquant_pack_roundtrip_and_sizes(L, fmt, n, k):
    w = synth.kquant_weights(synth.rng(n + k), fmt, n, k)
    buf = _kq_pack(w)
    high = {synth.Q5_K: k // 8, synth.Q6_K: k // 4}.get(fmt, 0)
    scale_row = {synth.Q4_K: 20, synth.Q5_K: 20, synth.Q6_K: 18, synth.IQ4_XS: 10}[fmt] * (k // 256)
    align = lambda v: (v + 255) // 256 * 256  # noqa: E731
    assert buf.nbytes == align(n * (k // 2 + high)) + align(n * scale_row) + 256
    assert qg.qg_scale_plane_offset(KQ[fmt], n, k) == align(n * (k // 2 + high))
    u = qg.qg_unpack_kquant(KQ[fmt], buf, n, k)
    for key, v in u.items():
        assert np.array_equal(v.view(np.uint8), np.asarray(w[key]).view(np.uint8)), key


@pytest.mark.parametrize("fmt", [synth.Q5_K, synth.Q6_K])
def test_kquant_high_bits_sit_one_byte_apart(L, fmt):
    """The documented placement: for dword q of a block's 4-bit plane, one
    shift and one mask of the high-bit word give the high bits of elements
    4q..4q+3 (and of 16+4q..16+4q+3), one per byte."""
    n, k = 3, 512
    w = synth.kquant_weights(synth.rng(5), fmt, n, k)
    buf = _kq_pack(w)
    row = k // 2 + (k // 8 if fmt == synth.Q5_K else k // 4)
    for r in range(n):
        base = r * row + k // 2
        for b in range(k // 32):
            if fmt == synth.Q5_K:
                h0 = h1 = int(buf[base + 4 * b:base + 4 * b + 4].view(np.uint32)[0])
            else:
                h0, h1 = (int(v) for v in buf[base + 8 * b:base + 8 * b + 8].view(np.uint32))
            for q in range(4):
                for i in range(4):
                    e_lo, e_hi = 32 * b + 4 * q + i, 32 * b + 16 + 4 * q + i
                    if fmt == synth.Q5_K:
                        lo, hi = (h0 >> q) >> (8 * i) & 1, (h1 >> (4 + q)) >> (8 * i) & 1
                    else:
                        lo, hi = (h0 >> (2 * q)) >> (8 * i) & 3, (h1 >> (2 * q)) >> (8 * i) & 3
                    assert lo == w["codes"][r, e_lo] >> 4 and hi == w["codes"][r, e_hi] >> 4


def test_kquant_argument_checks(L):
    w = synth.kquant_weights(synth.rng(6), synth.Q4_K, 2, 256)
    bad = dict(w, codes=w["codes"].copy())
    bad["codes"][1, 7] = 16
    with pytest.raises(qg.QGError):
        _kq_pack(bad)  # Q4_K code out of range
    bad = dict(w, sub=w["sub"].copy())
    bad["sub"][0, 3] = 64
    with pytest.raises(qg.QGError):
        _kq_pack(bad)  # 6-bit scale out of range
    with pytest.raises(qg.QGError):
        qg.qg_pack_kquant(qg.QG_Q4_K, w["codes"], w["d"], w["sub"])  # Q4_K needs dmin and mins
    assert qg.qg_packed_bytes(qg.QG_Q6_K, 4, 224) == 0  # k % 256
    w6 = synth.kquant_weights(synth.rng(7), synth.Q6_K, 2, 256)
    w6["sub"][:] = -128  # any int8 is a valid Q6_K scale
    _kq_pack(w6)
    assert L.qgemv_kquant_a8(qg.QG_Q4_0, 256, 4, 256, 256, 256, 256, 1, 256, None) == qg.QG_EINVAL  # format
    assert L.qgemv_kquant_a8(qg.QG_Q4_K, 256, 4, 224, 256, 256, 256, 1, 256, None) == qg.QG_EINVAL  # k % 256
    assert L.qgemv_kquant_a8(qg.QG_Q4_K, 256, 4, 256, 256, 256, None, 1, 256, None) == qg.QG_EINVAL  # xs required
    assert L.qgemv_kquant_a8(qg.QG_Q4_K, 256, 4, 256, 256, 256, 256, 17, 256, None) == qg.QG_EUNSUPPORTED


def test_prefill_a8_argument_checks(L):
    assert L.qgemm_prefill_a8(0, 4, 64, 256, 256, 1, 256, None) == qg.QG_EINVAL          # null w
    assert L.qgemm_prefill_a8(256, 4, 48, 256, 256, 1, 256, None) == qg.QG_EINVAL        # k % 32
    assert L.qgemm_prefill_a8(256, 4, 64, 256, 256, 0, 256, None) == qg.QG_EINVAL        # m < 1
    assert L.qgemm_prefill_a8(264, 4, 64, 256, 256, 1, 256, None) == qg.QG_EINVAL        # w misaligned
    assert L.qgemm_prefill_a8(256, 4, 64, 256, 256, 1 << 25, 256, None) == qg.QG_EUNSUPPORTED


def test_new_entry_points_reject_empty_and_null(L):
    """Zero tokens, zero rows and null activation scales are argument errors
    (checked on the host before anything is enqueued)."""
    assert L.qgemv_kquant_a8(qg.QG_Q6_K, 256, 4, 256, 256, 256, 256, 0, 256, None) == qg.QG_EINVAL  # m = 0
    assert L.qgemv_kquant_a8(qg.QG_Q6_K, 256, 0, 256, 256, 256, 256, 1, 256, None) == qg.QG_EINVAL  # n = 0
    assert L.qgemv_kquant_a8(qg.QG_IQ4_XS, 256, 4, 256, 256, None, 256, 1, 256, None) == qg.QG_EINVAL  # xd
    assert L.qgemm_prefill_a8(256, 0, 64, 256, 256, 4, 256, None) == qg.QG_EINVAL  # n = 0
    assert L.qgemm_prefill_a8(256, 4, 64, 256, None, 4, 256, None) == qg.QG_EINVAL  # xd
    assert L.qgemm_prefill_a8(256, 4, 64, 256, 256, 4, None, None) == qg.QG_EINVAL  # y
    for fmt in qg.KQUANT_FORMATS:
        assert qg.qg_packed_bytes(fmt, 1, 128) == 0 and qg.qg_packed_bytes(fmt, 1, 256) > 0


# ---------------------------------------------------------------- layout stamp and version


def _packed_examples():
    """(format code for qg_packed_check, n, k, packed buffer, unpack call) of every packer."""
    g = synth.rng(77)
    nv, q4, q8 = synth.nvfp4_weights(g, 3, 64), synth.q4_0_weights(g, 3, 64), synth.q8_0_weights(g, 3, 64)
    f8 = synth.fp8_weights(g, 3, 64, tiled=True)
    kq = synth.kquant_weights(g, synth.Q5_K, 2, 256)
    return [
        (qg.QG_NVFP4, 3, 64, qg.qg_pack_nvfp4(nv["codes"], nv["scales"]), lambda b: qg.qg_unpack_nvfp4(b, 3, 64)),
        (qg.QG_NVFP4_GATE_UP, 4, 64, qg.qg_pack_nvfp4_gate_up(nv["codes"][:2].repeat(2, 0), nv["scales"][:2].repeat(2, 0)),
         lambda b: qg.qg_unpack_nvfp4_gate_up(b, 2, 64)),
        (qg.QG_Q4_0, 3, 64, qg.qg_pack_q4_0(q4["codes"], q4["scales"]), lambda b: qg.qg_unpack_q4_0(b, 3, 64)),
        (qg.QG_Q8_0, 3, 64, qg.qg_pack_q8_0(q8["codes"], q8["scales"]), lambda b: qg.qg_unpack_q8_0(b, 3, 64)),
        (qg.QG_FP8_B128, 3, 64, qg.qg_pack_fp8(qg.QG_FP8_B128, f8["codes"], f8["scales"]),
         lambda b: qg.qg_unpack_fp8(qg.QG_FP8_B128, b, 3, 64)),
        (qg.QG_Q5_K, 2, 256, _kq_pack(kq), lambda b: qg.qg_unpack_kquant(qg.QG_Q5_K, b, 2, 256)),
    ]


def test_stamp_is_as_documented(L):
    for fmt, n, k, buf, _ in _packed_examples():
        st_ = buf[-256:]
        assert st_[:4].tobytes() == b"QGPK"
        v, f, kind = (int(x) for x in st_[4:16].view(np.uint32))
        assert v == qg.QG_LAYOUT_VERSION
        assert (f, kind) == ((qg.QG_NVFP4, 1) if fmt == qg.QG_NVFP4_GATE_UP else (fmt, 0))
        assert st_[16:32].view(np.int64).tolist() == [n, k] and not st_[32:].any()
        assert qg.qg_packed_check(fmt, buf, n, k) == qg.QG_OK


def test_other_layout_versions_are_rejected(L):
    """A buffer stamped by another layout version: QG_EVERSION from every
    unpacker and from qg_packed_check, before anything is read."""
    for fmt, n, k, buf, unpack in _packed_examples():
        for version in (1, qg.QG_LAYOUT_VERSION + 1):
            old = buf.copy()
            old[-256 + 4:-256 + 8] = np.array([version], np.uint32).view(np.uint8)
            assert qg.qg_packed_check(fmt, old, n, k) == qg.QG_EVERSION
            with pytest.raises(qg.QGError) as e:
                unpack(old)
            assert e.value.status == qg.QG_EVERSION


def test_unstamped_or_mismatched_buffers_are_rejected(L):
    for fmt, n, k, buf, unpack in _packed_examples():
        bare = buf.copy()
        bare[-256:] = 0  # no stamp (e.g. the previous layout, which had none)
        assert qg.qg_packed_check(fmt, bare, n, k) == qg.QG_EINVAL
        with pytest.raises(qg.QGError) as e:
            unpack(bare)
        assert e.value.status == qg.QG_EINVAL
        assert qg.qg_packed_check(fmt, buf[:-256], n, k) == qg.QG_ENOSPC
    nv = _packed_examples()[0][3]
    gu = _packed_examples()[1][3]
    assert qg.qg_packed_check(qg.QG_Q8_0, nv, 3, 64) != qg.QG_OK       # another format
    assert qg.qg_packed_check(qg.QG_NVFP4, gu, 4, 64) == qg.QG_EINVAL  # gate/up row order
    assert qg.qg_packed_check(qg.QG_NVFP4_GATE_UP, nv, 4, 64) == qg.QG_EINVAL
    with pytest.raises(qg.QGError):
        qg.qg_unpack_nvfp4(gu, 4, 64)                                     # plain unpack of gate/up
    big = np.concatenate([nv, np.zeros(4096, np.uint8)])
    assert qg.qg_packed_check(qg.QG_NVFP4, big, 3, 64) == qg.QG_OK       # larger buffers are fine
    assert qg.qg_packed_check(qg.QG_NVFP4, nv, 2, 64) != qg.QG_OK        # another shape


def test_moe_entry_points_reject_other_layout_versions(L):
    """Every MoE entry point takes packed experts through qg_moe_desc; a
    descriptor of another layout version is refused before any launch."""
    for version in (0, 1, qg.QG_LAYOUT_VERSION + 1):
        d = _desc(layout_version=version)
        assert qg.moe_workspace_bytes(d, 1) == 0
        assert qg.moe_prefill_workspace_bytes(d, 64) == 0
        r = ctypes.byref(d)
        assert L.moe_gemv_grouped(r, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 1 << 30, None) == qg.QG_EVERSION
        assert L.moe_forward(r, FAKE, FAKE, 1, FAKE, FAKE, 1 << 30, None) == qg.QG_EVERSION
        assert L.moe_forward_noalloc(r, FAKE, FAKE, 1, FAKE, None) == qg.QG_EVERSION
        assert L.moe_prefill(r, FAKE, FAKE, 64, FAKE, FAKE, 1 << 30, None) == qg.QG_EVERSION
    assert qg.moe_workspace_bytes(_desc(), 1) > 0
    assert qg.moe_workspace_bytes(_desc(reserved=1), 1) == 0


def test_noalloc_size_limit_on_host(L):
    """moe_forward_noalloc refuses a layer whose workspace exceeds its array
    (QG_ENOSPC) before touching the GPU."""
    d = _desc(hidden=8192, inter=4096, flags=qg.QG_MOE_KEEP_H,
              gate_up_stride=qg.qg_packed_bytes(qg.QG_NVFP4, 8192, 8192),
              down_stride=qg.qg_packed_bytes(qg.QG_NVFP4, 8192, 4096))
    assert qg.moe_workspace_bytes(d, 16) > qg.QG_MOE_NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(d), FAKE, FAKE, 16, FAKE, None) == qg.QG_ENOSPC
    assert L.moe_forward_noalloc(ctypes.byref(_desc()), FAKE, FAKE, 0, FAKE, None) == qg.QG_EINVAL
    assert L.moe_forward_noalloc(ctypes.byref(_desc()), FAKE, FAKE, 17, FAKE, None) == qg.QG_EUNSUPPORTED


def test_kernel_policy_seam():
    """qg_set_kernel_policy / qg_kernel_policy: the two documented values,
    QG_EINVAL for anything else (the policy unchanged), and QG_FORCE_KERNEL
    read once at first use (in a fresh process)."""
    import subprocess
    import sys

    try:
        assert qg.qg_kernel_policy() == qg.QG_KERNEL_TUNED
        qg.qg_set_kernel_policy(qg.QG_KERNEL_GENERIC)
        assert qg.qg_kernel_policy() == qg.QG_KERNEL_GENERIC
        for bad in (-1, 2, 99):
            assert qg.lib().qg_set_kernel_policy(bad) == qg.QG_EINVAL
            assert qg.qg_kernel_policy() == qg.QG_KERNEL_GENERIC
        qg.qg_set_kernel_policy(qg.QG_KERNEL_TUNED)
        assert qg.qg_kernel_policy() == qg.QG_KERNEL_TUNED
    finally:
        qg.qg_set_kernel_policy(qg.QG_KERNEL_TUNED)
    code = "import moe_expert_gemv_amd as qg; print(qg.qg_kernel_policy())"
    for env, want in (("generic", 1), ("tuned", 0), ("GENERIC", 0), ("", 0)):
        out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True,
                             env={**os.environ, "QG_FORCE_KERNEL": env}, cwd=ROOT)
        assert int(out.stdout.strip()) == want, env
