"""GPU parity at the full sizes of the measured workloads, every output
checked (the pages' gate runs every quant kernel against a CPU reference: bw24
README and memra README, correctness gates).

Each call is launched exactly as the benchmark launches it; the oracle is
evaluated in row (or column) chunks so that the fp64 dequantized weights never
exceed a few hundred MB at a time.
"""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.gpu_util import assert_within, dev, empty, host, pack_dev, pack_dev_gate_up, require_gpu

pytestmark = pytest.mark.gpu

CHUNK = 2048


def _gemv_chunked(w, x, n, fn_ref, fn_abs):
    ref = np.empty((x.shape[0], n))
    ab = np.empty_like(ref)
    for r0 in range(0, n, CHUNK):
        rows = np.arange(r0, min(r0 + CHUNK, n))
        ref[:, rows] = fn_ref(w, x, rows)
        ab[:, rows] = fn_abs(w, x, rows)
    return ref, ab


@pytest.mark.parametrize("m", [1, 4])
def test_dense_layer_every_output(m):
    """9B-class dense MLP (fused gate+up 24576 x 4096 + SwiGLU, down 4096 x
    12288), batch 1 and 4: every h, every a (from the GPU's own h) and every y
    (from the GPU's own a); each token bitwise equal to its batch-1 call."""
    import torch

    require_gpu()
    print(f"[full dense layer m={m}]", flush=True)
    L = synth.nvfp4_layer_case(m=m)
    inter, hidden = 12288, 4096
    wgu, wdn = pack_dev_gate_up(L.gate_up), pack_dev(L.down)
    x = dev(L.x)
    a = empty((m, inter), torch.int16)
    h = empty((m, 2 * inter), torch.float32)
    y = empty((m, hidden), torch.float32)
    qg.qgemv_nvfp4_swiglu(wgu, 0.01, inter, hidden, x, m, a, h)
    qg.qgemv_nvfp4(wdn, 0.01, hidden, inter, a, m, y)
    a_bits, hh, yy = host(a).view(np.uint16), host(h), host(y)
    ref, ab = _gemv_chunked(L.gate_up, L.x, 2 * inter, oracle.gemv, oracle.gemv_abs)
    assert_within(hh, ref, ab, f"gate+up h, all {2 * inter} rows, m={m}")
    exact = oracle.swiglu(hh.astype(np.float64))
    assert np.all(np.abs(oracle.decode_bf16(a_bits) - exact) <= oracle.bf16_ulp(exact)), "SwiGLU"
    ref, ab = _gemv_chunked(L.down, a_bits, hidden, oracle.gemv, oracle.gemv_abs)
    assert_within(yy, ref, ab, f"down y, all {hidden} rows, m={m}")
    if m > 1:
        for t in range(m):
            a1 = empty((1, inter), torch.int16)
            h1 = empty((1, 2 * inter), torch.float32)
            y1 = empty((1, hidden), torch.float32)
            qg.qgemv_nvfp4_swiglu(wgu, 0.01, inter, hidden, dev(L.x[t:t + 1]), 1, a1, h1)
            qg.qgemv_nvfp4(wdn, 0.01, hidden, inter, dev(a_bits[t:t + 1]), 1, y1)
            assert np.array_equal(host(h1).view(np.uint32), hh[t:t + 1].view(np.uint32)), t
            assert np.array_equal(host(a1).view(np.uint16), a_bits[t:t + 1]), t
            assert np.array_equal(host(y1).view(np.uint32), yy[t:t + 1].view(np.uint32)), t


@pytest.mark.parametrize("m", [1, 4])
def test_w4a8_every_output(m):
    """27B-class Q4_0 [17408 x 5120] x Q8_0 activations, batch 1 and 4: the
    quantizer bit-exact, every output within tolerance."""
    import torch

    require_gpu()
    print(f"[full w4a8 m={m}]", flush=True)
    case = synth.w4a8_case(m=m)
    n, k = case.w["codes"].shape
    xq = empty((m, k), torch.int8)
    xd = empty((m, k // 32), torch.int16)
    xs = empty((m, k // 32), torch.int32)
    y = empty((m, n), torch.float32)
    qg.qg_quantize_q8_0_act(dev(case.x), m, k, xq, xd, xs)
    qg.qgemv_q4_0_a8(pack_dev(case.w), n, k, xq, xd, xs, m, y)
    rq, rd, rs = oracle.quantize_q8_0_act(case.x)
    assert np.array_equal(host(xq), rq) and np.array_equal(host(xd).view(np.uint16), rd)
    assert np.array_equal(host(xs), rs)
    got = host(y)
    ref = np.empty((m, n))
    ab = np.empty_like(ref)
    for r0 in range(0, n, CHUNK):
        rows = np.arange(r0, min(r0 + CHUNK, n))
        ref[:, rows] = oracle.gemv_q4_0_a8(case.w, rq, rd, rows)
        ab[:, rows] = oracle.gemv_q4_0_a8_abs(case.w, rq, rd, rows)
    assert_within(got, ref, ab, f"w4a8 all {n} rows, m={m}")


def _prefill_check(w, x, got_bits, what):
    n = w["codes"].shape[0]
    got = oracle.decode_bf16(got_bits)
    rounded = 0
    for c0 in range(0, n, CHUNK):
        cols = np.arange(c0, min(c0 + CHUNK, n))
        ref, absum = oracle.prefill(w, x, cols=cols)
        tol = 1e-5 * absum + 1e-6 + oracle.bf16_ulp(ref)
        err = np.abs(got[:, cols] - ref)
        bad = ~(err <= tol)
        assert not bad.any(), f"{what} cols {c0}..: {bad.sum()} outside; worst {np.max(err / tol):.3f}"
        rounded += int(np.sum(got[:, cols] == oracle.round_to_bf16(ref)))
    # most outputs are the correctly rounded value of the exact result
    assert rounded / got.size > 0.97, what


@pytest.mark.parametrize("m,ws", [(64, True), (128, True), (512, False), (64, False), (128, False)])
def test_prefill_every_output(m, ws):
    """X bf16 [m x 4096] times the 9B-class NVFP4 [12288 x 4096]: every output
    of the workspace path (m <= 128, as measured) and of the single-pass path."""
    import torch

    require_gpu()
    print(f"[full prefill m={m} ws={ws}]", flush=True)
    case = synth.prefill_case(m=m)
    n, k = case.w["codes"].shape
    y = empty((m, n), torch.int16)
    w, x = pack_dev(case.w), dev(case.x)
    if ws:
        nbytes = qg.qgemm_prefill_workspace_bytes(n, k, m)
        buf = empty((max(nbytes, 256) // 4,), torch.float32)
        qg.qgemm_prefill_ws(w, 0.01, n, k, x, m, y, buf, nbytes)
    else:
        qg.qgemm_prefill(w, 0.01, n, k, x, m, y)
    _prefill_check(case.w, case.x, host(y).view(np.uint16), f"prefill m={m} ws={ws}")
