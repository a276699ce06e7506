"""GPU parity of the W4A8 prefill on the matrix cores (Q4_0 x Q8_0, int8
MFMA, exact int32 block dots, fp32 scale steps) against the W4A8 oracle:
shapes that span token and row tiles, ragged edges and one or two chunks of
activation scales, exact integer sums, batch invariance, and the 27B-class
projection at 512 tokens."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.gpu_util import assert_within, empty, host, pack_dev, require_gpu
from tests.test_gpu_a8 import quantize_gpu

pytestmark = pytest.mark.gpu


def run_pa8(w, xq, xd):
    import torch

    n, k = w["codes"].shape
    m = xq.shape[0]
    y = empty((m, n), torch.float32)
    qg.qgemm_prefill_a8(pack_dev(w), n, k, xq, xd, m, y)
    return host(y)


@pytest.mark.parametrize("n,k,m", [(1, 32, 1), (5, 64, 3), (130, 160, 17), (129, 4128, 65), (300, 512, 200),
                                   (64, 8192, 64), (17, 96, 130), (257, 5120, 129)])
def test_random(n, k, m):
    require_gpu()
    print(f"[prefill_a8 n={n} k={k} m={m}]", flush=True)
    g = synth.rng(n * 31 + k + m)
    w = synth.q4_0_weights(g, n, k)
    x = synth.x_f32(g, m, k)
    xq, xd, _ = quantize_gpu(x)
    rq, rd, _ = oracle.quantize_q8_0_act(x)
    assert_within(run_pa8(w, xq, xd), oracle.gemv_q4_0_a8(w, rq, rd), oracle.gemv_q4_0_a8_abs(w, rq, rd),
                  f"prefill_a8 {n}x{k} m={m}")


def test_integer_block_dots_are_exact():
    """d_w = 1 and integer x with a 127 in every block: d_x = 1, q_x = x, and
    y is the exact integer sum of the int32 block dots (every partial sum is
    below 2^24)."""
    require_gpu()
    g = synth.rng(51)
    n, k, m = 200, 512, 70
    w = synth.q4_0_weights(g, n, k)
    w["scales"][:] = 0x3C00
    x = g.integers(-127, 128, size=(m, k)).astype(np.float32)
    x[:, ::32] = 127.0
    xq, xd, _ = quantize_gpu(x)
    isum = oracle.block_isums_q4_0_a8(w, x.astype(np.int8))
    assert np.array_equal(run_pa8(w, xq, xd), isum.sum(axis=2).astype(np.float32))


def test_tokens_are_independent():
    """Each output depends only on its token: the rows of a 150-token call
    equal, bit for bit, calls on one token and on a 70-token slice."""
    require_gpu()
    g = synth.rng(52)
    w = synth.q4_0_weights(g, 300, 2048)
    x = synth.x_f32(g, 150, 2048)
    xq, xd, _ = quantize_gpu(x)
    y = run_pa8(w, xq, xd)
    for lo, hi in ((0, 1), (77, 78), (149, 150), (40, 110)):
        q1, d1, _ = quantize_gpu(x[lo:hi])
        assert np.array_equal(run_pa8(w, q1, d1).view(np.uint32), y[lo:hi].view(np.uint32))


def test_192_row_tile_matches_oracle_and_128_row_tile():
    """A grid of 128-row tiles that would need more than one round of
    resident workgroups (here 97 token blocks x 8 row blocks) runs on 192-row
    tiles: every output against the oracle (ragged rows, tokens and k stage),
    and token slices (128-row tiles) bitwise equal."""
    require_gpu()
    g = synth.rng(53)
    n, k, m = 1000, 160, 6200
    w = synth.q4_0_weights(g, n, k)
    x = synth.x_f32(g, m, k)
    xq, xd, _ = quantize_gpu(x)
    y = run_pa8(w, xq, xd)
    rq, rd, _ = oracle.quantize_q8_0_act(x)
    assert_within(y, oracle.gemv_q4_0_a8(w, rq, rd), oracle.gemv_q4_0_a8_abs(w, rq, rd), "prefill_a8 192-row tile")
    for lo, hi in ((0, 64), (3001, 3130), (6150, 6200)):
        q1, d1, _ = quantize_gpu(x[lo:hi])
        assert np.array_equal(run_pa8(w, q1, d1).view(np.uint32), y[lo:hi].view(np.uint32)), (lo, hi)


def test_full_size_512_tokens_sampled():
    """27B-class projection [17408 x 5120] over 512 tokens, sampled rows."""
    require_gpu()
    print("[prefill_a8 full]", flush=True)
    case = synth.w4a8_case(m=512)
    xq, xd, _ = quantize_gpu(case.x)
    got = run_pa8(case.w, xq, xd)
    rq, rd, _ = oracle.quantize_q8_0_act(case.x)
    n = case.w["codes"].shape[0]
    rows = np.unique(np.concatenate([np.arange(4), np.arange(n - 4, n), synth.rng(3).integers(0, n, 88)]))
    assert_within(got[:, rows], oracle.gemv_q4_0_a8(case.w, rq, rd, rows),
                  oracle.gemv_q4_0_a8_abs(case.w, rq, rd, rows), "prefill_a8 full")
