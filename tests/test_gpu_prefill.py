"""GPU parity of the small-M prefill GEMM (NVFP4 weights, bf16 activations,
matrix cores, bf16 output)."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.conftest import load_golden
from tests.gpu_util import dev, empty, host, pack_dev, require_gpu

pytestmark = pytest.mark.gpu


def run_prefill(w, x_bits):
    import torch

    n, k = w["codes"].shape
    m = x_bits.shape[0]
    y = empty((m, n), torch.int16)
    qg.qgemm_prefill(pack_dev(w), float(w["tensor_scale"]), n, k, dev(x_bits), m, y)
    return host(y).view(np.uint16)


def run_prefill_ws(w, x_bits):
    """The workspace variant (k split over workgroups for m <= 128 with k not
    a multiple of 256)."""
    import torch

    n, k = w["codes"].shape
    m = x_bits.shape[0]
    y = empty((m, n), torch.int16)
    nbytes = qg.qgemm_prefill_workspace_bytes(n, k, m)
    ws = empty((max(nbytes, 256) // 4,), torch.float32)
    qg.qgemm_prefill_ws(pack_dev(w), float(w["tensor_scale"]), n, k, dev(x_bits), m, y, ws, nbytes)
    return host(y).view(np.uint16)


def check(w, x, rows=None, cols=None, what="", run=run_prefill):
    got_bits = run(w, x)
    if rows is not None:
        got_bits = got_bits[np.ix_(rows, cols)]
    got = oracle.decode_bf16(got_bits)
    ref, absum = oracle.prefill(w, x, rows, cols)
    tol = 1e-5 * absum + 1e-6 + oracle.bf16_ulp(ref)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside; worst {np.max(err / tol):.3f}"
    # most outputs are the correctly rounded value of the exact result
    assert np.mean(got == oracle.round_to_bf16(ref)) > 0.97, what


def test_worked_example():
    require_gpu()
    ex6 = next(e for e in load_golden("worked_examples.json")["examples"] if e["id"] == "EX-6")
    ex9 = next(e for e in load_golden("worked_examples.json")["examples"] if e["id"] == "EX-9")
    w = {"fmt": "nvfp4", "codes": np.array(ex6["codes"], np.uint8), "scales": np.array(ex6["scales"], np.uint8),
         "tensor_scale": np.float32(ex6["tensor_scale"])}
    X = np.zeros((2, 32), np.float32)
    X[0] = 1.0
    X[1, 20] = 1.0
    got = oracle.decode_bf16(run_prefill(w, synth.to_bf16_bits(X)))
    assert got.tolist() == ex9["Y"]


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (3, 17, 64), (64, 64, 64), (65, 130, 96), (100, 300, 512),
                                   (128, 64, 4096), (7, 1000, 2080), (513, 129, 160),
                                   # M <= 128, k a multiple of 256 (one-pass kernel): 1 to 14 stages of
                                   # 256 (whole rounds of four and the tails), ragged n, one and two
                                   # token blocks
                                   (1, 47, 256), (64, 97, 768), (65, 48, 1280), (128, 145, 2304), (33, 50, 3584),
                                   # M > 128, k a multiple of 256 (eight-wave kernel), ragged m and n
                                   (129, 193, 256), (300, 200, 768), (257, 385, 2048),
                                   # M > 128, other k (four-wave kernel)
                                   (200, 100, 1056)])
def test_random(m, n, k):
    require_gpu()
    print(f"[prefill m={m} n={n} k={k}]", flush=True)
    g = synth.rng(m * 7 + n * 3 + k)
    w = synth.nvfp4_weights(g, n, k)
    x = synth.x_bf16(g, m, k)
    check(w, x, what=f"prefill {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (3, 17, 64), (64, 64, 64), (65, 130, 96), (100, 300, 512),
                                   (128, 200, 4096), (7, 1000, 2080), (37, 193, 1056), (128, 385, 3072),
                                   (513, 129, 160)])
def test_random_workspace(m, n, k):
    """qgemm_prefill_ws: k slices of 1024 (a partial last slice, a k tail
    inside a slice), rows of 64, columns of 192 with ragged ends."""
    require_gpu()
    print(f"[prefill ws m={m} n={n} k={k}]", flush=True)
    g = synth.rng(m * 11 + n * 5 + k)
    w = synth.nvfp4_weights(g, n, k)
    x = synth.x_bf16(g, m, k)
    check(w, x, what=f"prefill ws {m}x{n}x{k}", run=run_prefill_ws)


@pytest.mark.parametrize("m,n,k", [(64, 100, 1024), (128, 49, 768)])
def test_workspace_path_is_one_pass_for_whole_stages(m, n, k):
    """With k a multiple of 256 the workspace variant is qgemm_prefill itself
    (no workspace; bitwise the same result)."""
    require_gpu()
    print(f"[prefill ws one-pass m={m} n={n} k={k}]", flush=True)
    assert qg.qgemm_prefill_workspace_bytes(n, k, m) == 0
    g = synth.rng(m + n + k)
    w = synth.nvfp4_weights(g, n, k)
    x = synth.x_bf16(g, m, k)
    assert np.array_equal(run_prefill_ws(w, x), run_prefill(w, x))


def test_workspace_rows_are_independent():
    """With the workspace, a row's result does not depend on the other rows
    or on m (m <= 128)."""
    require_gpu()
    g = synth.rng(19)
    w = synth.nvfp4_weights(g, 256, 2080)
    x = synth.x_bf16(g, 128, 2080)
    full = run_prefill_ws(w, x)
    assert np.array_equal(run_prefill_ws(w, x[64:65]), full[64:65])
    assert np.array_equal(run_prefill_ws(w, x[:5]), full[:5])
    assert np.array_equal(run_prefill_ws(w, x[27:127]), full[27:127])


def test_one_hot_rows_are_exact():
    require_gpu()
    g = synth.rng(8)
    n, k = 96, 256
    w = synth.nvfp4_weights(g, n, k, tensor_scale=1.0)
    cols = [0, 15, 16, 31, 100, 255]
    X = np.zeros((len(cols), k), np.float32)
    for i, c in enumerate(cols):
        X[i, c] = 1.0
    got = oracle.decode_bf16(run_prefill(w, synth.to_bf16_bits(X)))
    D = oracle.dequant_nvfp4(w)
    for i, c in enumerate(cols):
        assert np.array_equal(got[i], D[:, c])  # e2m1 * e4m3 is exact in bf16


def test_rows_are_independent():
    """A row's result does not depend on the other rows of the batch, nor on
    M inside each shape (M <= 128; M > 128, here with k a multiple of 256);
    across shapes results agree to rounding (the parity tests)."""
    require_gpu()
    g = synth.rng(9)
    w = synth.nvfp4_weights(g, 256, 1024)
    x = synth.x_bf16(g, 260, 1024)
    small = run_prefill(w, x[:100])
    assert np.array_equal(run_prefill(w, x[64:65]), small[64:65])
    assert np.array_equal(run_prefill(w, x[:5]), small[:5])
    assert np.array_equal(run_prefill(w, x[36:128])[:64], small[36:100])
    large = run_prefill(w, x)
    assert np.array_equal(run_prefill(w, x[1:130]), large[1:130])
    assert np.array_equal(run_prefill(w, x[100:260]), large[100:260])


