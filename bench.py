#!/usr/bin/env python3
"""Benchmark of the block-quantized decode GEMV path on one MI355X.

Default workload: one batch-1 decode step of a 9B-class dense MLP with NVFP4
weights -- fused gate+up GEMV [24576 x 4096] with the SwiGLU epilogue, then
the down GEMV [4096 x 12288] -- on seeded synthetic weights.  A step is both
kernels.  The metric is achieved HBM bandwidth over the algorithmic bytes
(packed codes + scales once, activations in, outputs out).

Measurement:
  * the weights exist in R copies (>= 1 GiB in total) and step i uses copy
    i mod R, so no step finds its weights in the 256 MB Infinity Cache or L2;
  * warmup and timed steps each run as one HIP-graph replay (the pages' decode
    is one graph replay per token); the timed replay is bracketed by
    synchronisations and HIP events;
  * the dominant kernel is timed alone: a graph of back-to-back launches of it
    (on rotating weight copies) replayed on its own stream between two HIP
    events; the launch duration is the region divided by the launch count;
  * the CPU baseline is the oracle (fp64 numpy, one thread) running whole
    steps of the same workload for a bounded time.

Prints one JSON line.  ``--config`` selects the other workloads (Q8_0, W4A8,
MoE, prefill) for design measurements.

Two CPU-only modes turn rocprofv3 output (rocpd SQLite databases) into the
text summaries and the per-launch HBM traffic kept with the sources:
  ``--summarize-rocprof DB --command CMD``: per-kernel duration table;
  ``--write-traffic --config C --fetch-db F --write-db W``: FETCH_SIZE and
  WRITE_SIZE of the workload's dominant kernel(s), each scaled by what the same
  counter read for the plain copy that ``--calibrate-copy`` adds to a run.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized GEMV achieved HBM GB/s (% of ~8 TB/s) + µs/call, batch 1"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_INT8_TOPS = 5000.0
ROTATE_BYTES = 1 << 30


CSRC = "moe_expert_gemv_amd/csrc"
_COMMON_SOURCES = ("qg_device.hpp", "qg_layout.hpp")
COPY_CAL_BYTES = 256 << 20  # the plain copy that calibrates the byte counters


def _code_only(text: str) -> str:
    """Source text without comments and blank lines (edits to comments do not
    change the kernel a counter summary was taken on)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_digest(files) -> str:
    """Digest of the code of the sources a kernel is built from (its .hip file,
    the headers it includes); a committed counter summary is valid only for
    that digest."""
    h = hashlib.sha256()
    for name in sorted(set(files) | set(_COMMON_SOURCES)):
        with open(os.path.join(ROOT, CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


PROFILES = {  # config -> its rocprofv3 summary under profiles/
    "dense": "nvfp4_gemv__dense_layer_h4096_i12288_m1", "dense-m4": "nvfp4_gemv__dense_layer_h4096_i12288_m4",
    "q8": "q8_0_gemv__1024x1024_m1", "w4a8": "q4_0_a8_gemv__17408x5120_m1",
    "w4a8-m4": "q4_0_a8_gemv__17408x5120_m4", "fp8": "fp8_gemv__24576x4096_block128_m1",
    "q4k": "q4_k_a8_gemv__17408x5120_m1", "q5k": "q5_k_a8_gemv__17408x5120_m1",
    "q6k": "q6_k_a8_gemv__17408x5120_m1", "iq4xs": "iq4_xs_a8_gemv__17408x5120_m1",
    "moe": "moe_gate_up_down__e256_h2048_i512_top8_t1", "moe-t4": "moe_gate_up_down__e256_h2048_i512_top8_t4",
    "moe-prefill": "moe_prefill_grouped_mfma__e256_h2048_i512_top8_t512",
    "prefill64": "prefill_mfma__12288x4096_m64", "prefill128": "prefill_mfma__12288x4096_m128",
    "prefill512": "prefill_mfma__12288x4096_m512",
    "w4a8-prefill512": "q4_0_a8_prefill_int8_mfma__17408x5120_m512",
    "probe-read": "probe_read__1GiB_streaming", "probe-mfma": "probe_mfma__bf16_16x16x32",
}


def kernel_trace_from_profile(config: str, cls) -> dict | None:
    """The dominant launch's mean duration in the committed rocprofv3 kernel
    trace of this config (sum over its kernels of their mean durations), or
    None when there is no summary or it was taken on other kernel sources."""
    name = PROFILES.get(config)
    path = os.path.join(ROOT, "profiles", f"{name}.txt") if name else None
    if not path or not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel sources digest ([0-9a-f]+)", text)
    if not m or m.group(1) != source_digest(cls.sources):
        return None
    total = 0.0
    for pat in cls.kernel_re:
        rows = [ln for ln in text.splitlines() if re.match(r"\s*\d+\s+[\d.]+", ln) and re.search(pat, ln)]
        if not rows:
            return None
        total += sum(float(r.split()[1]) for r in rows)
    return {"us_per_launch": total, "file": f"profiles/{name}.txt"}


def traffic_from_profile(config: str, cls) -> int | None:
    """HBM bytes per dominant launch from profiles/traffic.json, or None when
    there is no entry or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(config)
    if not ent or ent.get("source_digest") != source_digest(cls.sources):
        return None
    return ent.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- workloads

class Workload:
    name = ""
    dominant = ""
    bound = "hbm"
    mfma_peak = (PEAK_BF16_TFLOPS, "TFLOP/s")  # dense peak of the contraction's dtype
    sources: tuple = ()     # files under csrc/ the dominant kernel(s) are built from
    kernel_re: tuple = ()   # one dominant launch = one dispatch of each of these kernels

    def step(self, i: int):  # enqueue step i on the current stream
        raise NotImplementedError

    def dominant_launch(self, i: int):
        raise NotImplementedError

    # The CPU baseline: the oracle run on `cpu_parts` slices of the step (row
    # slices of the weights, or routings / token groups for MoE), one slice
    # at a time until the time budget is used; each slice reports the
    # algorithmic bytes of the step it accounts for.
    cpu_parts = 1
    has_oracle = True  # False for the chip probes, which have no oracle to time

    def cpu_part_desc(self) -> str:
        return f"the oracle on 1/{self.cpu_parts} of the weight rows"

    def cpu_part_steps(self) -> float:  # fraction of a step one part is
        return 1.0 / self.cpu_parts

    def cpu_sample(self, part: int, parts: int) -> float:
        raise NotImplementedError

    # also time the oracle on one thread (reported beside the all-core figure)
    cpu_single_thread = False

    def cpu_baseline(self, budget_s=12.0, threads=1):
        from threadpoolctl import threadpool_limits

        total, done, n = 0.0, 0.0, 0
        with threadpool_limits(limits=threads):
            while total < budget_s and n < 1_000_000:
                t1 = time.perf_counter()
                done += self.cpu_sample(n % self.cpu_parts, self.cpu_parts)
                total += time.perf_counter() - t1
                n += 1
        return {"value": done / total / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": f"{n} samples, each {self.cpu_part_desc()} ({n * self.cpu_part_steps():.3f} steps in "
                          f"all) in {total:.1f} s, fp64 numpy, BLAS on {threads} thread(s)"}


def host_cores() -> int:
    """CPU cores this process may run on (its affinity mask)."""
    return len(os.sched_getaffinity(0))


def blas_config() -> dict:
    """What the CPU baseline's matmuls run on: numpy's BLAS build and the
    thread pools threadpoolctl sees, plus OMP_NUM_THREADS."""
    from threadpoolctl import threadpool_info

    try:
        build = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {})
    except TypeError:  # older numpy: no dict mode
        build = {}
    pools = [{k: p.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer", "architecture")}
             for p in threadpool_info()]
    return {"numpy_blas": {k: build.get(k) for k in ("name", "version", "openblas configuration")},
            "thread_pools": pools, "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def _slice(part: int, parts: int, n: int) -> np.ndarray:
    return np.arange(part * n // parts, (part + 1) * n // parts)


def _copies(unit_bytes: int) -> int:
    return max(2, int(np.ceil(ROTATE_BYTES / unit_bytes)))


class DenseLayer(Workload):
    """gate+up [2I x H] + SwiGLU, then down [H x I], batch m."""

    sources = ("k_gemv_nvfp4.hip", "qg_gemv_core.hpp", "qg_mfma.hpp", "qg_reduce.hpp")
    # the SwiGLU instance: fourth template argument of the batch-1 kernel, fifth of the batched one
    kernel_re = (r"k_gemv_nvfp4_stream<(?:\d+, ){3}true\b|k_gemv_nvfp4<(?:\d+, ){4}true\b",)

    def __init__(self, m=1):
        import torch
        import moe_expert_gemv_amd as qg
        import synth

        self.qg = qg
        self.m = m
        self.H, self.I = 4096, 12288
        case = synth.nvfp4_layer_case(m=m)
        self.case = case
        gu = qg.qg_pack_nvfp4_gate_up(case.gate_up["codes"], case.gate_up["scales"])
        dn = qg.qg_pack_nvfp4(case.down["codes"], case.down["scales"])
        self.R = _copies(gu.nbytes + dn.nbytes)
        self.gu = torch.from_numpy(gu).cuda().repeat(self.R, 1)  # R x bytes, each row 256-B aligned
        self.dn = torch.from_numpy(dn).cuda().repeat(self.R, 1)
        assert gu.nbytes % 256 == 0 and dn.nbytes % 256 == 0
        self.x = torch.from_numpy(case.x.view(np.int16).copy()).cuda()
        self.a = torch.empty((m, self.I), dtype=torch.int16, device="cuda")
        self.y = torch.empty((m, self.H), dtype=torch.float32, device="cuda")
        H, I = self.H, self.I
        # algorithmic bytes: packed codes + scales, activations in, outputs out
        self.alg_gu = (2 * I) * (H // 2) + (2 * I) * (H // 16) + 2 * m * H + 2 * m * I
        self.alg_dn = H * (I // 2) + H * (I // 16) + 2 * m * I + 4 * m * H
        self.alg_step = self.alg_gu + self.alg_dn
        self.flops_step = 2 * m * (2 * I * H + H * I)
        self.name = (f"nvfp4 dense decode layer (9B-class): gate+up {2 * I}x{H} + SwiGLU, down {H}x{I}, "
                     f"bf16 activations, batch {m}")
        self.dominant = "gate+up GEMV with SwiGLU epilogue"
        self.dominant_bytes = self.alg_gu

    def _gate_up(self, i):
        self.qg.qgemv_nvfp4_swiglu(self.gu[i % self.R], 0.01, self.I, self.H, self.x, self.m, self.a, None)

    def step(self, i):
        self._gate_up(i)
        self.qg.qgemv_nvfp4(self.dn[i % self.R], 0.01, self.H, self.I, self.a, self.m, self.y)

    def dominant_launch(self, i):
        self._gate_up(i)

    def cpu_baseline(self, budget_s=12.0, threads=1):
        """The oracle running whole decode steps of this layer (fp64 numpy
        dequantize + dot, the matmuls on `threads` BLAS threads), repeated
        until the time budget is used; throughput over the same algorithmic
        bytes as the GPU step."""
        import oracle
        from threadpoolctl import threadpool_limits

        case = self.case
        H, I = self.H, self.I
        chunk = 2048
        total, done_bytes, steps = 0.0, 0, 0
        with threadpool_limits(limits=threads):
            while total < budget_s:
                t1 = time.perf_counter()
                a = np.empty((self.m, I))
                for r0 in range(0, I, chunk):
                    r = np.arange(r0, min(r0 + chunk, I))
                    h = oracle.gemv(case.gate_up, case.x, np.concatenate([r, r + I]))
                    a[:, r] = oracle.swiglu_bf16(h)
                for r0 in range(0, H, chunk):
                    oracle.gemv(case.down, a, np.arange(r0, min(r0 + chunk, H)))
                total += time.perf_counter() - t1
                done_bytes += self.alg_step
                steps += 1
        return {"value": done_bytes / total / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": f"{steps} whole decode steps of the same layer (gate+up, SwiGLU, down) "
                          f"in {total:.1f} s, fp64 numpy, BLAS on {threads} thread(s)"}


class Q8Gemv(Workload):
    sources = ("k_gemv_q8.hip",)
    kernel_re = (r"k_gemv_q8_0\b",)
    cpu_single_thread = True

    def __init__(self, m=1):
        import torch
        import moe_expert_gemv_amd as qg
        import synth

        self.qg, self.m = qg, m
        case = synth.q8_gemv_case(m=m)
        self.case = case
        buf = qg.qg_pack_q8_0(case.w["codes"], case.w["scales"])
        self.R = _copies(buf.nbytes)
        self.w = torch.from_numpy(buf).cuda().repeat(self.R, 1)
        self.x = torch.from_numpy(case.x).cuda()
        self.y = torch.empty((m, 1024), dtype=torch.float32, device="cuda")
        self.alg_step = 1024 * 1024 + 1024 * 32 * 2 + 4 * m * 1024 * 2
        self.dominant_bytes = self.alg_step
        self.flops_step = 2 * m * 1024 * 1024
        self.name = f"q8_0 GEMV 1024x1024, fp32 activations, batch {m}"
        self.dominant = "Q8_0 GEMV"

    cpu_parts = 4

    def cpu_sample(self, part, parts):
        import oracle

        rows = _slice(part, parts, 1024)
        oracle.gemv(self.case.w, self.case.x, rows)
        return self.alg_step * len(rows) / 1024

    def step(self, i):
        self.qg.qgemv_q8_0(self.w[i % self.R], 1024, 1024, self.x, self.m, self.y)

    dominant_launch = step


class Fp8Gemv(Workload):
    """FP8 E4M3 weight GEMV with block-128 scales at the gate+up shape of the
    9B-class layer (the pages' 9B model runs FP8 weights)."""

    sources = ("k_gemv_fp8.hip",)
    kernel_re = (r"k_gemv_fp8\b",)

    def __init__(self, m=1):
        import torch
        import moe_expert_gemv_amd as qg
        import synth

        self.qg, self.m = qg, m
        self.N, self.K = 24576, 4096
        g = synth.rng(synth.seed_for(6))
        w = synth.fp8_weights(g, self.N, self.K, tiled=True)
        buf = qg.qg_pack_fp8(qg.QG_FP8_B128, w["codes"], w["scales"])
        self.R = _copies(buf.nbytes)
        self.w = torch.from_numpy(buf).cuda().repeat(self.R, 1)
        x = synth.x_bf16(g, m, self.K)
        self.w_log, self.x_log = w, x
        self.x = torch.from_numpy(x.view(np.int16).copy()).cuda()
        self.y = torch.empty((m, self.N), dtype=torch.float32, device="cuda")
        scales = w["scales"].size * 4
        self.alg_step = self.N * self.K + scales + 2 * m * self.K + 4 * m * self.N
        self.dominant_bytes = self.alg_step
        self.flops_step = 2 * m * self.N * self.K
        self.name = (f"FP8 E4M3 GEMV {self.N}x{self.K} (9B-class gate+up), block-128 fp32 scales, "
                     f"bf16 activations, batch {m}")
        self.dominant = "FP8 GEMV"

    cpu_parts = 24

    def cpu_sample(self, part, parts):
        import oracle

        rows = _slice(part, parts, self.N)
        oracle.gemv(self.w_log, self.x_log, rows)
        return self.alg_step * len(rows) / self.N

    def step(self, i):
        self.qg.qgemv_fp8(self.qg.QG_FP8_B128, self.w[i % self.R], self.N, self.K, self.x, self.m, self.y)

    dominant_launch = step


class W4A8Gemv(Workload):
    sources = ("k_gemv_a8.hip", "qg_mfma.hpp", "qg_reduce.hpp")
    kernel_re = (r"k_gemv_q4_0_a8\b",)
    cpu_single_thread = True

    def __init__(self, m=1):
        import torch
        import moe_expert_gemv_amd as qg
        import synth

        self.qg, self.m = qg, m
        self.N, self.K = 17408, 5120
        case = synth.w4a8_case(m=m)
        self.case = case
        buf = qg.qg_pack_q4_0(case.w["codes"], case.w["scales"])
        self.R = _copies(buf.nbytes)
        self.w = torch.from_numpy(buf).cuda().repeat(self.R, 1)
        self.x = torch.from_numpy(case.x).cuda()
        K = self.K
        self.xq = torch.empty((m, K), dtype=torch.int8, device="cuda")
        self.xd = torch.empty((m, K // 32), dtype=torch.int16, device="cuda")
        self.xs = torch.empty((m, K // 32), dtype=torch.int32, device="cuda")
        self.y = torch.empty((m, self.N), dtype=torch.float32, device="cuda")
        N = self.N
        self.dominant_bytes = N * K // 2 + N * (K // 32) * 2 + m * (K + K // 32 * 6) + 4 * m * N
        self.alg_step = self.dominant_bytes + m * K * 4 + m * (K + K // 32 * 6)
        self.flops_step = 2 * m * N * K
        self.name = f"q4_0 x q8_0 (W4A8) GEMV {N}x{K} (27B-class), batch {m}"
        self.dominant = "W4A8 GEMV"

    cpu_parts = 17

    def cpu_sample(self, part, parts):
        import oracle

        rows = _slice(part, parts, self.N)
        xq, xd, _ = oracle.quantize_q8_0_act(self.case.x)
        oracle.gemv_q4_0_a8(self.case.w, xq, xd, rows)
        return self.alg_step * len(rows) / self.N

    def step(self, i):
        self.qg.qg_quantize_q8_0_act(self.x, self.m, self.K, self.xq, self.xd, self.xs)
        self.dominant_launch(i)

    def dominant_launch(self, i):
        self.qg.qgemv_q4_0_a8(self.w[i % self.R], self.N, self.K, self.xq, self.xd, self.xs, self.m, self.y)


class KQuantGemv(Workload):
    """K-quant / IQ4_XS weights x Q8_0 activations at the 27B-class
    projection shape [17408 x 5120] (the shape the pages' 27B runs in Q4_K /
    Q5_K / Q6_K use)."""
    sources = ("k_gemv_kquant.hip",)
    kernel_re = (r"k_gemv_kquant\b",)
    fmt = ""

    def __init__(self, m=1):
        import torch
        import moe_expert_gemv_amd as qg
        import synth

        self.qg, self.m = qg, m
        self.N, self.K = 17408, 5120
        self.code = {"q4_k": qg.QG_Q4_K, "q5_k": qg.QG_Q5_K, "q6_k": qg.QG_Q6_K, "iq4_xs": qg.QG_IQ4_XS}[self.fmt]
        case = synth.kquant_case(self.fmt, m=m)
        self.case = case
        w = case.w
        buf = qg.qg_pack_kquant(self.code, w["codes"], w["d"], w["sub"], w.get("dmin"), w.get("mins"))
        self.R = _copies(buf.nbytes)
        self.w = torch.from_numpy(buf).cuda().repeat(self.R, 1)
        self.x = torch.from_numpy(case.x).cuda()
        N, K = self.N, self.K
        self.xq = torch.empty((m, K), dtype=torch.int8, device="cuda")
        self.xd = torch.empty((m, K // 32), dtype=torch.int16, device="cuda")
        self.xs = torch.empty((m, K // 32), dtype=torch.int32, device="cuda")
        self.y = torch.empty((m, N), dtype=torch.float32, device="cuda")
        # packed codes + scales (bytes of the layout, not of its padding)
        high = {"q5_k": K // 8, "q6_k": K // 4}.get(self.fmt, 0)
        srow = {"q4_k": 20, "q5_k": 20, "q6_k": 18, "iq4_xs": 10}[self.fmt] * (K // 256)
        self.dominant_bytes = N * (K // 2 + high + srow) + m * (K + K // 32 * 6) + 4 * m * N
        self.alg_step = self.dominant_bytes + m * K * 4 + m * (K + K // 32 * 6)
        self.flops_step = 2 * m * N * K
        self.name = f"{self.fmt} x q8_0 GEMV {N}x{K} (27B-class), batch {m}"
        self.dominant = f"{self.fmt} GEMV"

    cpu_parts = 17

    def cpu_sample(self, part, parts):
        import oracle

        rows = _slice(part, parts, self.N)
        xq, xd, _ = oracle.quantize_q8_0_act(self.case.x)
        oracle.gemv_a8(self.case.w, xq, xd, rows)
        return self.alg_step * len(rows) / self.N

    def step(self, i):
        self.qg.qg_quantize_q8_0_act(self.x, self.m, self.K, self.xq, self.xd, self.xs)
        self.dominant_launch(i)

    def dominant_launch(self, i):
        self.qg.qgemv_kquant_a8(self.code, self.w[i % self.R], self.N, self.K, self.xq, self.xd, self.xs, self.m,
                                self.y)


class Q4KGemv(KQuantGemv):
    fmt = "q4_k"


class Q5KGemv(KQuantGemv):
    fmt = "q5_k"


class Q6KGemv(KQuantGemv):
    fmt = "q6_k"


class IQ4XSGemv(KQuantGemv):
    fmt = "iq4_xs"


class MoE(Workload):
    sources = ("k_moe.hip", "qg_gemv_core.hpp")
    kernel_re = (r"k_moe_gate_up(?:_tile)?\b", r"k_moe_down(?:_tile)?\b")

    routing_samples = 64  # routings drawn (one per step, cycled)

    def __init__(self, t=1):
        import torch
        import moe_expert_gemv_amd as qg
        import oracle
        import synth

        self.qg, self.t = qg, t
        L = synth.moe_case(t=t)
        E = L.n_experts + 1
        H, I = L.hidden, L.inter
        gs = qg.qg_packed_bytes(qg.QG_NVFP4, 2 * I, H)
        ds = qg.qg_packed_bytes(qg.QG_NVFP4, H, I)
        gu = np.concatenate([qg.qg_pack_nvfp4_gate_up(L.gate_up[e]["codes"], L.gate_up[e]["scales"])
                             for e in range(E)])
        dn = np.concatenate([qg.qg_pack_nvfp4(L.down[e]["codes"], L.down[e]["scales"]) for e in range(E)])
        self.R = _copies(gu.nbytes + dn.nbytes)
        self.gu = torch.from_numpy(gu).cuda().repeat(self.R, 1)
        self.dn = torch.from_numpy(dn).cuda().repeat(self.R, 1)
        self.gs, self.ds = gs, ds
        self.scales = torch.full((E,), 0.01, dtype=torch.float32, device="cuda")
        self.L = L
        # a fresh routing per step (logits drawn per step) so steps touch different experts
        self.S = self.routing_samples
        g = synth.rng(synth.seed_for(4, 900))
        logits = synth.logits_f32(g, self.S * t, L.n_experts)
        self.logits_np = logits.reshape(self.S, t, L.n_experts)
        self.logits = torch.from_numpy(logits).cuda().view(self.S, t, L.n_experts)
        self.x = torch.from_numpy(L.x.view(np.int16).copy()).cuda()
        self.ids = torch.empty((t, 8), dtype=torch.int32, device="cuda")
        self.w = torch.empty((t, 8), dtype=torch.float32, device="cuda")
        self.y = torch.empty((t, H), dtype=torch.float32, device="cuda")
        self.descs = []
        for r in range(self.R):
            d = qg.QgMoeDesc(n_experts=256, top_k=8, has_shared=1, flags=0, hidden=H, inter=I,
                             gate_up=self.gu[r].data_ptr(), gate_up_stride=gs, down=self.dn[r].data_ptr(),
                             down_stride=ds, gate_up_scale=self.scales.data_ptr(),
                             down_scale=self.scales.data_ptr())
            self.descs.append(d)
        self.ws_bytes = self.workspace_bytes(self.descs[0], t)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device="cuda")
        # algorithmic bytes: the active experts' packed weights + activations
        u = []
        for s in range(self.S):
            ids, _ = oracle.route_topk(logits.reshape(self.S, t, -1)[s], 8)
            u.append(len(set(ids.ravel().tolist())) + 1)
        self.mean_active = float(np.mean(u))
        self.alg_step = int(self.mean_active * (2 * I * H * 9 // 16 + H * I * 9 // 16)) + t * (2 * H + 4 * H)
        self.dominant_bytes = self.alg_step  # the dominant launch is the whole moe_forward call
        self.flops_step = int(2 * t * 9 * (2 * I * H + H * I))
        self.name = (f"moe decode (35B-A3B-like): 256 routed + 1 shared experts, hidden {H}, inter {I}, "
                     f"top-8, {t} token(s), routing drawn per step")
        self.dominant = "moe_forward: routing + grouped gate/up + SwiGLU, grouped down + combine (2 kernels)"

    def workspace_bytes(self, desc, t):
        return self.qg.moe_workspace_bytes(desc, t)

    @property
    def cpu_parts(self):
        return self.S

    def cpu_part_desc(self):
        return "one whole step (the oracle's routing, grouping, gate/up, SwiGLU, down and combine) with its own routing"

    def cpu_part_steps(self):
        return 1.0

    def _moe_bytes(self, ids, t):
        H, I = self.L.hidden, self.L.inter
        active = len(set(np.asarray(ids).ravel().tolist())) + 1
        return active * (2 * I * H * 9 // 16 + H * I * 9 // 16) + t * (2 * H + 4 * H)

    def cpu_sample(self, part, parts):
        import oracle

        ids, wts = oracle.route_topk(self.logits_np[part], 8)
        oracle.moe_forward(self.L, self.L.x, ids, wts)
        return self._moe_bytes(ids, self.t)

    def step(self, i):
        # routing + grouped expert GEMVs + combine: two launches
        self.qg.moe_forward(self.descs[i % self.R], self.x, self.logits[i % self.S], self.t, self.y, self.ws,
                            self.ws_bytes)

    dominant_launch = step


class MoEPrefill(MoE):
    """The same layer over a prompt of t tokens (grouped NVFP4 MoE GEMM on the
    matrix cores): at t = 512 every expert is active, so a step streams all
    257 experts' weights once."""

    sources = ("k_moe_prefill.hip", "k_moe.hip", "qg_mfma.hpp")
    kernel_re = (r"k_route_topk\b", r"k_mpf_place\b", r"k_mpf_gemm\w*<[^>]*\btrue>",
                 r"k_mpf_gemm\w*<[^>]*\bfalse>", r"k_mpf_combine\b")
    routing_samples = 8

    def __init__(self, t=512):
        super().__init__(t)
        self.name = (f"moe prefill (35B-A3B-like): 256 routed + 1 shared experts, hidden {self.L.hidden}, "
                     f"inter {self.L.inter}, top-8, {t} tokens, routing drawn per step")
        self.dominant = "moe_prefill: routing, grouping, grouped gate/up + SwiGLU and down GEMMs, combine (5 kernels)"

    def workspace_bytes(self, desc, t):
        return self.qg.moe_prefill_workspace_bytes(desc, t)

    cpu_tokens = 8

    @property
    def cpu_parts(self):
        return self.t // self.cpu_tokens

    def cpu_part_desc(self):
        return (f"the oracle's layer for {self.cpu_tokens} of the {self.t} tokens (bytes: the experts they select, "
                f"each once, and their activations)")

    def cpu_part_steps(self):
        return self.cpu_tokens / self.t

    def cpu_sample(self, part, parts):
        import oracle

        tok = _slice(part, parts, self.t)
        ids, wts = oracle.route_topk(self.logits_np[0][tok], 8)
        oracle.moe_forward(self.L, self.L.x[tok], ids, wts)
        return self._moe_bytes(ids, len(tok))

    def step(self, i):
        self.qg.moe_prefill(self.descs[i % self.R], self.x, self.logits[i % self.S], self.t, self.y, self.ws,
                            self.ws_bytes)

    dominant_launch = step


class Prefill(Workload):
    sources = ("k_prefill.hip", "qg_mfma.hpp")
    kernel_re = (r"k_prefill(8|_sm)?\b",)

    def __init__(self, m=512):
        import torch
        import moe_expert_gemv_amd as qg
        import synth

        self.qg, self.m = qg, m
        self.N, self.K = 12288, 4096
        case = synth.prefill_case(m=m)
        self.case = case
        buf = qg.qg_pack_nvfp4(case.w["codes"], case.w["scales"])
        self.R = _copies(buf.nbytes)
        self.w = torch.from_numpy(buf).cuda().repeat(self.R, 1)
        self.x = torch.from_numpy(case.x.view(np.int16).copy()).cuda()
        self.y = torch.empty((m, self.N), dtype=torch.int16, device="cuda")
        N, K = self.N, self.K
        self.alg_step = N * K * 9 // 16 + 2 * m * K + 2 * m * N
        self.dominant_bytes = self.alg_step
        self.flops_step = 2 * m * N * K
        self.bound = "mfma" if m >= 96 else "hbm"
        self.name = f"prefill GEMM: X bf16 [{m}x{K}] x NVFP4 W [{N}x{K}], bf16 out"
        self.dominant = "prefill MFMA GEMM"

    cpu_parts = 96

    def cpu_sample(self, part, parts):
        import oracle

        cols = _slice(part, parts, self.N)
        oracle.prefill(self.case.w, self.case.x, cols=cols)
        return self.alg_step * len(cols) / self.N

    def step(self, i):
        self.qg.qgemm_prefill(self.w[i % self.R], 0.01, self.N, self.K, self.x, self.m, self.y)

    dominant_launch = step


class PrefillA8(Workload):
    """W4A8 prefill on the int8 matrix cores: Q8_0-quantized fp32 activations
    [m x 5120] times the 27B-class Q4_0 projection [17408 x 5120], fp32 out."""
    sources = ("k_prefill_a8.hip", "qg_mfma.hpp")
    kernel_re = (r"k_prefill_a8\b",)
    bound = "mfma"
    mfma_peak = (PEAK_INT8_TOPS, "TOP/s")

    def __init__(self, m=512):
        import torch
        import moe_expert_gemv_amd as qg
        import synth

        self.qg, self.m = qg, m
        self.N, self.K = 17408, 5120
        case = synth.w4a8_case(m=m)
        self.case = case
        buf = qg.qg_pack_q4_0(case.w["codes"], case.w["scales"])
        self.R = _copies(buf.nbytes)
        self.w = torch.from_numpy(buf).cuda().repeat(self.R, 1)
        self.x = torch.from_numpy(case.x).cuda()
        N, K = self.N, self.K
        self.xq = torch.empty((m, K), dtype=torch.int8, device="cuda")
        self.xd = torch.empty((m, K // 32), dtype=torch.int16, device="cuda")
        self.y = torch.empty((m, N), dtype=torch.float32, device="cuda")
        self.dominant_bytes = N * K // 2 + N * (K // 32) * 2 + m * (K + K // 32 * 2) + 4 * m * N
        self.alg_step = self.dominant_bytes + m * K * 4 + m * (K + K // 32 * 2)
        self.flops_step = 2 * m * N * K
        self.name = f"W4A8 prefill (int8 MFMA): q8_0 X [{m}x{K}] x q4_0 W [{N}x{K}] (27B-class), fp32 out"
        self.dominant = "W4A8 prefill int8 MFMA GEMM"

    cpu_parts = 272

    def cpu_sample(self, part, parts):
        import oracle

        rows = _slice(part, parts, self.N)
        xq, xd, _ = oracle.quantize_q8_0_act(self.case.x)
        oracle.gemv_q4_0_a8(self.case.w, xq, xd, rows)
        return self.alg_step * len(rows) / self.N

    def step(self, i):
        self.qg.qg_quantize_q8_0_act(self.x, self.m, self.K, self.xq, self.xd, None)
        self.dominant_launch(i)

    def dominant_launch(self, i):
        self.qg.qgemm_prefill_a8(self.w[i % self.R], self.N, self.K, self.xq, self.xd, self.m, self.y)


class ProbeRead(Workload):
    """Achievable HBM read bandwidth: the library's streaming-read probe
    (16-byte non-temporal loads, 1 KB per wave-wide load, eight in flight per
    lane) over copies of `nbytes` that rotate through at least 1 GiB (four
    times the 256 MB Infinity Cache), at the workgroups-per-CU count that
    reads fastest here.  At 1 GiB the launch ramp is negligible; at a
    kernel's own byte count it is what a plain read of those bytes costs."""
    has_oracle = False
    sources = ("k_probe.hip", "qg_mfma.hpp")
    kernel_re = (r"k_probe_read\b",)
    cpu_parts = 1

    def __init__(self, nbytes=1 << 30):
        import torch
        import moe_expert_gemv_amd as qg

        self.qg = qg
        self.bytes = max(16, nbytes // 16 * 16)
        self.R = max(2, -(-(1 << 30) // self.bytes))
        self.bufs = torch.full((self.R, self.bytes), 7, dtype=torch.uint8, device="cuda")
        self.sink = torch.zeros(64, dtype=torch.int32, device="cuda")
        self.wg = best_read_probe_shape(self.bufs[0], self.sink)
        self.alg_step = self.dominant_bytes = self.bytes
        self.flops_step = 0
        size = f"{self.bytes >> 30} GiB" if self.bytes % (1 << 30) == 0 else f"{self.bytes / 1e6:.1f} MB"
        self.name = (f"streaming-read probe: {size} per launch over {self.R} rotating copies, "
                     f"{self.wg} four-wave workgroup(s) per CU")
        self.dominant = "streaming-read probe"

    def step(self, i):
        self.qg.qg_probe_read(self.bufs[i % self.R], self.wg, self.sink)

    dominant_launch = step


class ProbeMfma(Workload):
    """Achievable dense bf16 MFMA rate: v_mfma_f32_16x16x32_bf16 with sixteen
    independent accumulators per wave, two waves per SIMD."""
    has_oracle = False
    sources = ("k_probe.hip", "qg_mfma.hpp")
    kernel_re = (r"k_probe_mfma\b",)
    bound = "mfma"
    cpu_parts = 1

    def __init__(self, iters=4000):
        import torch
        import moe_expert_gemv_amd as qg

        self.qg, self.iters = qg, iters
        self.sink = torch.zeros(64, dtype=torch.float32, device="cuda")
        self.flops_step = qg.qg_probe_mfma_bf16(iters, self.sink)
        torch.cuda.synchronize()
        self.alg_step = self.dominant_bytes = 0
        self.name = f"bf16 MFMA probe: {iters} rounds of 16 independent 16x16x32 MFMAs per wave, 8 waves per CU"
        self.dominant = "bf16 MFMA probe"

    def step(self, i):
        self.qg.qg_probe_mfma_bf16(self.iters, self.sink)

    dominant_launch = step


def best_read_probe_shape(buf, sink, shapes=(1, 2, 4)) -> int:
    """Workgroups per CU at which the read probe streams fastest (a short sweep)."""
    import torch
    import moe_expert_gemv_amd as qg

    best, best_t = shapes[0], float("inf")
    for wg in shapes:
        qg.qg_probe_read(buf, wg, sink)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            qg.qg_probe_read(buf, wg, sink)
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b)
        if t < best_t:
            best, best_t = wg, t
    return best


def achievable_peaks(bound: str, launch_bytes: int = 0) -> dict:
    """What this GPU reaches with the probes: read GB/s for HBM-bound
    configs, bf16 MFMA TFLOP/s for matrix-core-bound ones (graph replays of
    the probe between two HIP events, best of three).  For HBM-bound configs
    also the read probe at the dominant launch's own byte count, whose ramp
    and drain a one-shot GEMV pays as well."""
    if bound != "hbm":
        wl = ProbeMfma()
        _, mean = time_dominant(wl, 8)
        return {"bf16_mfma_tflops": wl.flops_step / (mean * 1e-3) / 1e12, "probe": wl.name}
    wl = ProbeRead()
    _, mean = time_dominant(wl, 8)
    out = {"read_gbs": wl.bytes / (mean * 1e-3) / 1e9, "probe": wl.name}
    del wl
    if launch_bytes:
        wl = ProbeRead(launch_bytes)
        _, mean = time_dominant(wl, min(wl.R, 32))
        out["at_launch_bytes"] = {"us": mean * 1e3, "read_gbs": wl.bytes / (mean * 1e-3) / 1e9, "probe": wl.name}
    return out


CONFIGS = {  # name -> (workload class, its size argument)
    "dense": (DenseLayer, 1),
    "dense-m4": (DenseLayer, 4),
    "q8": (Q8Gemv, 1),
    "w4a8": (W4A8Gemv, 1),
    "w4a8-m4": (W4A8Gemv, 4),
    "fp8": (Fp8Gemv, 1),
    "q4k": (Q4KGemv, 1),
    "q5k": (Q5KGemv, 1),
    "q6k": (Q6KGemv, 1),
    "iq4xs": (IQ4XSGemv, 1),
    "moe": (MoE, 1),
    "moe-t4": (MoE, 4),
    "moe-prefill": (MoEPrefill, 512),
    "prefill64": (Prefill, 64),
    "prefill128": (Prefill, 128),
    "prefill512": (Prefill, 512),
    "w4a8-prefill512": (PrefillA8, 512),
    "probe-read": (ProbeRead, 1 << 30),
    "probe-mfma": (ProbeMfma, 4000),
}


# ---------------------------------------------------------------- timing

def _blocker(stream):
    """Keep the GPU busy ~2 ms so the CPU can queue work ahead of it."""
    import torch

    with torch.cuda.stream(stream):
        a = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(6):
            b.copy_(a)
    return a, b


def time_steps(wl: Workload, steps: int, warmup: int, use_graph: bool):
    import torch

    stream = torch.cuda.Stream()
    if use_graph:
        with torch.cuda.stream(stream):
            wl.step(0)  # first eager call outside capture
        torch.cuda.synchronize()
        gw = torch.cuda.CUDAGraph()
        gt = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=stream):
            for i in range(warmup):
                wl.step(i)
        with torch.cuda.graph(gt, stream=stream):
            for i in range(steps):
                wl.step(warmup + i)
        run_w, run_t = gw.replay, gt.replay
    else:
        def run_w():
            for i in range(warmup):
                wl.step(i)

        def run_t():
            for i in range(steps):
                wl.step(warmup + i)

    with torch.cuda.stream(stream):
        run_w()
    torch.cuda.synchronize()
    keep = _blocker(stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0.record(stream)
        run_t()
        t1.record(stream)
    torch.cuda.synchronize()
    del keep
    return t0.elapsed_time(t1) / steps  # ms per step


def time_dominant(wl: Workload, launches: int, reps: int = 3):
    """Average duration of one dominant launch: a graph of `launches`
    back-to-back launches (rotating weight copies) replayed on its own stream
    between two HIP events recorded on that stream; best of `reps` replays."""
    import torch

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        wl.dominant_launch(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(launches):
            wl.dominant_launch(i + 1)
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        keep = _blocker(stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        del keep
        per.append(a.elapsed_time(b) / launches)  # ms
    return float(min(per)), float(np.mean(per))


def calibrate_copy():
    """A plain device copy of COPY_CAL_BYTES (fp32 negation: every byte read
    once, written once), run three times; the byte counters of a profiled run
    are scaled by what they read for this kernel."""
    import torch

    n = COPY_CAL_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        flush.zero_()  # evict src from L2 / Infinity Cache
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- rocprofv3 summaries

def _dispatches(db: str):
    """(kernel display name, duration ns) of every dispatch in a rocpd database."""
    import sqlite3

    c = sqlite3.connect(db)
    q = ("SELECT S.display_name, K.end - K.start FROM rocpd_kernel_dispatch K "
         "JOIN rocpd_info_kernel_symbol S ON S.id = K.kernel_id AND S.guid = K.guid")
    return c.execute(q).fetchall()


def _short(name: str) -> str:
    name = name.replace("void ", "", 1) if name.startswith("void ") else name
    name = name.replace("qg::(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in name:  # drop the argument list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out)[:110]


def summarize_rocprof(db: str, command: str) -> str:
    by = {}
    for name, ns in _dispatches(db):
        by.setdefault(name, []).append(ns / 1e3)
    total = sum(sum(v) for v in by.values())
    lines = ["rocprofv3 kernel trace summary (durations in microseconds)",
             f"command: {command}", "",
             f"{'calls':>6} {'avg':>9} {'median':>9} {'min':>9} {'max':>9} {'total%':>7}  kernel"]
    for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(v)
        lines.append(f"{len(a):6d} {a.mean():9.2f} {np.median(a):9.2f} {a.min():9.2f} {a.max():9.2f} "
                     f"{100 * a.sum() / total:7.2f}  {_short(name)}")
    return "\n".join(lines) + "\n"


def _counter_avgs(db: str, counter: str, pattern: str):
    """Mean counter value (KiB per dispatch) over dispatches whose name matches."""
    import re
    import sqlite3

    c = sqlite3.connect(db)
    rows = c.execute("SELECT kernel_name, dispatch_id, SUM(value) FROM counters_collection "
                     "WHERE counter_name = ? GROUP BY dispatch_id, kernel_name", (counter,)).fetchall()
    v = [val for name, _, val in rows if re.search(pattern, name)]
    if not v:
        raise SystemExit(f"no dispatch of /{pattern}/ with {counter} in {db}")
    return float(np.mean(v)), len(v)


def write_traffic(config: str, fetch_db: str, write_db: str, command: str):
    cls = CONFIGS[config][0]
    cal_kib = COPY_CAL_BYTES / 1024
    f_cal, _ = _counter_avgs(fetch_db, "FETCH_SIZE", r"neg_kernel")
    w_cal, _ = _counter_avgs(write_db, "WRITE_SIZE", r"neg_kernel")
    f_scale, w_scale = cal_kib / f_cal, cal_kib / w_cal
    fetch = write = 0.0
    per_kernel = {}
    for pat in cls.kernel_re:
        f, nf = _counter_avgs(fetch_db, "FETCH_SIZE", pat)
        w, nw = _counter_avgs(write_db, "WRITE_SIZE", pat)
        per_kernel[pat] = {"fetch_kib_raw": f, "write_kib_raw": w, "dispatches": [nf, nw]}
        fetch += f * f_scale * 1024
        write += w * w_scale * 1024
    ent = {"kernels": per_kernel, "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_calibration_bytes": COPY_CAL_BYTES, "fetch_bytes_per_launch": int(round(fetch)),
           "write_bytes_per_launch": int(round(write)), "hbm_bytes_per_launch": int(round(fetch + write)),
           "source_digest": source_digest(cls.sources), "sources": list(cls.sources), "command": command}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[config] = ent
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({config: ent}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="dense", choices=sorted(CONFIGS))
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly instead of a graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the achievable-peak probe")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain copy of known size first (for byte-counter calibration)")
    ap.add_argument("--summarize-rocprof", metavar="DB", help="print a kernel summary of a rocpd database")
    ap.add_argument("--write-traffic", action="store_true", help="record the dominant kernel's HBM bytes")
    ap.add_argument("--fetch-db")
    ap.add_argument("--write-db")
    ap.add_argument("--command", default="", help="the profiled command, recorded with a summary")
    args = ap.parse_args()

    if args.summarize_rocprof:
        sys.stdout.write(summarize_rocprof(args.summarize_rocprof, args.command))
        return
    if args.write_traffic:
        write_traffic(args.config, args.fetch_db, args.write_db, args.command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode GEMV path runs on a single device (the "
              "multi-GPU sharding is a design note, not built); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import moe_expert_gemv_amd as qg

    qg.lib()
    print(f"[bench] building workload {args.config}", file=sys.stderr, flush=True)
    cls, size = CONFIGS[args.config]
    wl = cls(size)
    if args.calibrate_copy:
        calibrate_copy()
    print(f"[bench] {wl.name}; {getattr(wl, 'R', 1)} weight copies; timing", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    ms = time_steps(wl, args.steps, args.warmup, not args.no_graph)
    dom_best, dom_mean = time_dominant(wl, max(20, min(args.steps, 200)))
    value = wl.alg_step / (ms * 1e-3) / 1e9

    if wl.bound == "mfma":
        achieved = wl.flops_step / (dom_mean * 1e-3) / 1e12
        peak, unit = wl.mfma_peak
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak}
    else:
        achieved = wl.dominant_bytes / (dom_mean * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    roof["traffic"] = traffic_from_profile(args.config, cls)
    roof["kernel"] = wl.dominant
    # HIP events around a graph of back-to-back launches: the per-launch
    # period, i.e. the kernel plus the gap between two dependent launches
    roof["us_per_launch"] = dom_mean * 1e3
    roof["us_per_launch_best_replay"] = dom_best * 1e3
    roof["alg_bytes_per_launch"] = wl.dominant_bytes
    if not args.no_probe and not args.config.startswith("probe") and (
            wl.bound == "hbm" or wl.mfma_peak[0] == PEAK_BF16_TFLOPS):
        print("[bench] achievable peak (probe)", file=sys.stderr, flush=True)
        roof["achievable"] = achievable_peaks("hbm" if wl.bound == "hbm" else "mfma",
                                              wl.dominant_bytes if wl.bound == "hbm" else 0)
        ach = roof["achievable"].get("read_gbs") or roof["achievable"].get("bf16_mfma_tflops")
        roof["achievable"]["frac_of_achievable"] = roof["achieved"] / ach
        at = roof["achievable"].get("at_launch_bytes")
        if at:  # the same bytes by a plain read, against this launch
            at["frac_of_plain_read"] = roof["achieved"] / at["read_gbs"]
    kt = kernel_trace_from_profile(args.config, cls)
    if kt:  # the kernel alone, from the committed rocprofv3 trace of this command
        t_k = kt["us_per_launch"] * 1e-6
        roof["kernel_trace"] = dict(kt, frac=(wl.flops_step / t_k / 1e12 if wl.bound == "mfma"
                                              else wl.dominant_bytes / t_k / 1e9) / roof["peak"])

    cpu = None
    if not args.no_cpu_baseline and wl.has_oracle:
        cores = host_cores()
        print(f"[bench] timing the CPU oracle baseline on {cores} cores", file=sys.stderr, flush=True)
        cpu = wl.cpu_baseline(args.cpu_budget, cores)
        if wl.cpu_single_thread:
            print("[bench] timing the CPU oracle baseline on 1 thread", file=sys.stderr, flush=True)
            one = wl.cpu_baseline(args.cpu_budget, 1)
            cpu["single_thread"] = {"value": one["value"], "unit": one["unit"], "sample": one["sample"]}
        cpu["host_cores"] = cores
        cpu["blas"] = blas_config()

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_step": ms * 1e3,
        "pct_of_peak_hbm": 100.0 * value / PEAK_HBM_GBS,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generators; random codes/scales of the stated distributions)",
        "config": {"workload": wl.name, "alg_bytes_per_step": wl.alg_step,
                   "weight_copies_rotated": getattr(wl, "R", 1),
                   "graph_replay": not args.no_graph,
                   "kernel_source_digest": source_digest(cls.sources)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
