"""The kernel policy (the library's rollback seam): under QG_KERNEL_GENERIC
the calls that have a generic kernel take it, with the results the header
documents -- bitwise those of the tuned kernels for the NVFP4 GEMV at one
token and for the MoE layer at two to four tokens, and qgemm_prefill's for
qgemm_prefill_ws -- and within the oracle's tolerance."""
import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import oracle
import synth
from tests.gpu_util import assert_within, dev, empty, host, pack_dev, require_gpu
from tests.test_gpu_gemv import run_nvfp4
from tests.test_gpu_moe import Layer, check_moe, route_gpu, run_moe
from tests.test_gpu_prefill import check, run_prefill, run_prefill_ws
from tests.test_gpu_swiglu import run_swiglu

pytestmark = pytest.mark.gpu


@pytest.fixture
def policy():
    """Run a body under both policies; always back to the tuned one."""
    def run(policy_value, fn, *args):
        qg.qg_set_kernel_policy(policy_value)
        try:
            return fn(*args)
        finally:
            qg.qg_set_kernel_policy(qg.QG_KERNEL_TUNED)
    yield run
    qg.qg_set_kernel_policy(qg.QG_KERNEL_TUNED)


@pytest.mark.parametrize("n,k", [(333, 2048), (333, 4096), (129, 6144), (200, 12288), (64, 192)])
def test_nvfp4_one_token_generic_kernel(policy, n, k):
    require_gpu()
    print(f"[policy nvfp4 n={n} k={k}]", flush=True)
    g = synth.rng(n + k + 3)
    w = synth.nvfp4_weights(g, n, k)
    x = synth.x_bf16(g, 1, k)
    tuned = policy(qg.QG_KERNEL_TUNED, run_nvfp4, w, x)
    generic = policy(qg.QG_KERNEL_GENERIC, run_nvfp4, w, x)
    assert np.array_equal(tuned.view(np.uint32), generic.view(np.uint32))
    assert_within(generic, oracle.gemv(w, x), oracle.gemv_abs(w, x), "generic nvfp4")


@pytest.mark.parametrize("k", [4096, 12288])
def test_swiglu_one_token_generic_kernel(policy, k):
    require_gpu()
    g = synth.rng(k + 17)
    inter = 96
    w = synth.nvfp4_weights(g, 2 * inter, k)
    x = synth.x_bf16(g, 1, k)
    a_t, h_t = policy(qg.QG_KERNEL_TUNED, run_swiglu, w, x, inter)
    a_g, h_g = policy(qg.QG_KERNEL_GENERIC, run_swiglu, w, x, inter)
    assert np.array_equal(a_t, a_g) and np.array_equal(h_t.view(np.uint32), h_g.view(np.uint32))


@pytest.mark.parametrize("t", [2, 3, 4])
def test_moe_few_tokens_generic_kernels(policy, t):
    require_gpu()
    print(f"[policy moe t={t}]", flush=True)
    L = synth.moe_case(t=t, n_experts=32, top_k=8, hidden=2048, inter=512, has_shared=True, seed=700 + t)
    layer = Layer(L)
    ids_d, w_d = route_gpu(L.logits, 8)
    y_t, ws_t, _ = policy(qg.QG_KERNEL_TUNED, run_moe, layer, L.x, ids_d, w_d)
    y_g, ws_g, _ = policy(qg.QG_KERNEL_GENERIC, run_moe, layer, L.x, ids_d, w_d)
    assert np.array_equal(y_t.view(np.uint32), y_g.view(np.uint32))
    assert np.array_equal(ws_t, ws_g)  # CSR, a, h and o as well
    policy(qg.QG_KERNEL_GENERIC, check_moe, L, layer, t)


@pytest.mark.parametrize("m,n,k", [(64, 200, 4160), (100, 300, 2080), (128, 385, 3104)])
def test_prefill_ws_generic_is_single_pass(policy, m, n, k):
    require_gpu()
    print(f"[policy prefill_ws m={m} n={n} k={k}]", flush=True)
    g = synth.rng(m * 7 + n + k)
    w = synth.nvfp4_weights(g, n, k)
    x = synth.x_bf16(g, m, k)
    single = run_prefill(w, x)
    generic = policy(qg.QG_KERNEL_GENERIC, run_prefill_ws, w, x)
    assert np.array_equal(single, generic)
    policy(qg.QG_KERNEL_GENERIC, check, w, x, None, None, "generic prefill_ws", run_prefill_ws)
