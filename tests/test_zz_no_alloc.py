"""moe_forward_noalloc (the MoE layer with its workspace in the library's
own device array) against moe_forward with a caller workspace: bitwise equal
on two calls in a row, the second with fewer tokens and a different routing,
plus the host-side size limit."""
import ctypes

import numpy as np
import pytest

import moe_expert_gemv_amd as qg
import synth
from tests.gpu_util import dev, empty, host, require_gpu

pytestmark = pytest.mark.gpu


def _layer(t, seed):
    import torch

    L = synth.moe_case(t=t, n_experts=256, top_k=8, hidden=2048, inter=512, seed=seed)
    E = L.n_experts + 1
    gu = np.concatenate([qg.qg_pack_nvfp4_gate_up(L.gate_up[e]["codes"], L.gate_up[e]["scales"])
                         for e in range(E)])
    dn = np.concatenate([qg.qg_pack_nvfp4(L.down[e]["codes"], L.down[e]["scales"]) for e in range(E)])
    gud, dnd = dev(gu), dev(dn)
    sc = torch.full((E,), 0.01, dtype=torch.float32, device="cuda")
    d = qg.QgMoeDesc(n_experts=256, top_k=8, has_shared=1, flags=0, hidden=2048, inter=512,
                     gate_up=gud.data_ptr(), gate_up_stride=qg.qg_packed_bytes(qg.QG_NVFP4, 1024, 2048),
                     down=dnd.data_ptr(), down_stride=qg.qg_packed_bytes(qg.QG_NVFP4, 2048, 512),
                     gate_up_scale=sc.data_ptr(), down_scale=sc.data_ptr())
    return L, d, (gud, dnd, sc)


def _with_ws(d, x, logits, t):
    import torch

    y = empty((t, 2048), torch.float32)
    nb = qg.moe_workspace_bytes(d, t)
    ws = empty((nb,), torch.uint8)
    qg.moe_forward(d, x, logits, t, y, ws, nb)
    return host(y)


def test_noalloc_matches_workspace_call_twice():
    import torch

    require_gpu()
    L, d, keep = _layer(4, seed=9100)
    g = synth.rng(9101)
    for t in (4, 1):  # the second call is smaller
        print(f"[moe_forward_noalloc t={t}]", flush=True)
        x = dev(synth.x_bf16(g, t, 2048))
        logits = dev(synth.logits_f32(g, t, 256))
        ref = _with_ws(d, x, logits, t)
        y = empty((t, 2048), torch.float32)
        y.fill_(float("nan"))
        qg.moe_forward_noalloc(d, x, logits, t, y)
        got = host(y)
        assert np.all(np.isfinite(got))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), t


def test_noalloc_rejects_oversize_on_host():
    """A layer whose workspace exceeds the array: QG_ENOSPC before any launch."""
    require_gpu()
    d = qg.QgMoeDesc(n_experts=256, top_k=8, has_shared=1, flags=qg.QG_MOE_KEEP_H, hidden=8192, inter=4096,
                     gate_up=256, gate_up_stride=qg.qg_packed_bytes(qg.QG_NVFP4, 8192, 8192),
                     down=256, down_stride=qg.qg_packed_bytes(qg.QG_NVFP4, 8192, 4096),
                     gate_up_scale=256, down_scale=256)
    assert qg.moe_workspace_bytes(d, 16) > qg.QG_MOE_NOALLOC_SCRATCH_BYTES
    st = qg.lib().moe_forward_noalloc(ctypes.byref(d), 256, 256, 16, 256, None)
    assert st == -4  # QG_ENOSPC
