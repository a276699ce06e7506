"""Seeded synthetic inputs for the block-quantized GEMV path.

This module only draws random numbers and stores them in the raw encodings the
formats use (code bytes, E4M3 / fp16 / bf16 bit patterns).  It holds none of the
method's arithmetic: no decoding, no dot products, no quantization of
activations.  Encodings of the drawn floats into E4M3, fp16 and bf16 bit
patterns are done by library casts (``torch`` for E4M3 and bf16, numpy for fp16,
all round-to-nearest-even).

Both the CPU oracle (``oracle/``) and the GPU path's tests and benchmark read
their inputs from here, so the two sides always see identical bytes.

Workload shapes stand in for the decode layers of the models the source pages
benchmark (a 9B-class dense MLP, a 27B-class projection, a 35B-A3B-like MoE
layer); the distributions are:

* Q8_0 weights: int8 codes uniform in [-127, 127]; one fp16 scale per
  32-element block drawn as |N(0,1)| * 0.02 / 127.
* NVFP4 weights: E2M1 codes uniform over all 16 codes; one E4M3 scale per
  16-element block drawn as |N(0,1)| * 0.5 (rounded to E4M3); fp32 tensor
  scale 0.01.
* Q4_0 weights: 4-bit codes uniform in 0..15; one fp16 scale per 32-element
  block drawn as |N(0,1)| * 0.01.
* K-quant / IQ4_XS weights: see ``kquant_weights``.
* Activations: N(0,1), as fp32 or rounded to bf16.
* Router logits: fp32 N(0,1).

Seeds: ``seed_for(cfg, tensor_index)`` = 20261202 + 1000*cfg + tensor_index;
draw order inside one tensor set is codes, then scales, then activations, then
logits.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20261202

# Format tags shared by the generator output dicts (plain strings, no arithmetic).
NVFP4 = "nvfp4"
Q8_0 = "q8_0"
Q4_0 = "q4_0"
FP8 = "fp8"
FP8_TILE = 128  # side of an FP8 block-128 scale tile
Q4_K = "q4_k"
Q5_K = "q5_k"
Q6_K = "q6_k"
IQ4_XS = "iq4_xs"
KQ_SUPER = 256  # elements per super-block of the K-quant and IQ4_XS formats
KQUANTS = (Q4_K, Q5_K, Q6_K, IQ4_XS)


def seed_for(cfg: int, tensor_index: int = 0) -> int:
    return BASE_SEED + 1000 * cfg + tensor_index


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# raw encodings via library casts
# --------------------------------------------------------------------------

def to_e4m3_bits(v: np.ndarray) -> np.ndarray:
    """E4M3 (OCP 'FN') bytes of float values, rounded by torch's cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def to_f16_bits(v: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns of float values (numpy's RNE cast)."""
    return np.ascontiguousarray(v, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float values (torch's RNE cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


# --------------------------------------------------------------------------
# weight sets (logical form: one code per byte, row-major [n, k])
# --------------------------------------------------------------------------

def nvfp4_weights(g: np.random.Generator, n: int, k: int, tensor_scale: float = 0.01) -> dict:
    assert k % 16 == 0
    codes = g.integers(0, 16, size=(n, k), dtype=np.uint8)
    sc = np.abs(g.standard_normal(size=(n, k // 16))) * 0.5
    return {
        "fmt": NVFP4,
        "n": n,
        "k": k,
        "codes": codes,
        "scales": to_e4m3_bits(sc),
        "tensor_scale": np.float32(tensor_scale),
    }


def fp8_weights(g: np.random.Generator, n: int, k: int, tiled: bool = True, std: float = 0.02) -> dict:
    """FP8 E4M3 weights the way FP8 checkpoints are made: w ~ N(0, std) in
    fp32, one fp32 scale per 128 x 128 tile (tiled) or per tensor equal to the
    tile's max |w| / 448, codes = E4M3 of w / scale (torch's cast)."""
    w = (g.standard_normal(size=(n, k)) * std).astype(np.float32)
    if tiled:
        tn, tk = (n + FP8_TILE - 1) // FP8_TILE, (k + FP8_TILE - 1) // FP8_TILE
        pad = np.zeros((tn * FP8_TILE, tk * FP8_TILE), np.float32)
        pad[:n, :k] = np.abs(w)
        amax = pad.reshape(tn, FP8_TILE, tk, FP8_TILE).max(axis=(1, 3))
    else:
        amax = np.array([[np.abs(w).max()]], np.float32)
    scales = np.maximum(amax, np.float32(1e-30)).astype(np.float32) / np.float32(448.0)
    full = np.repeat(np.repeat(scales, FP8_TILE, axis=0), FP8_TILE, axis=1)[:n, :k] if tiled else scales[0, 0]
    codes = to_e4m3_bits(w / full)
    return {"fmt": FP8, "tiled": tiled, "n": n, "k": k, "codes": codes, "scales": scales.astype(np.float32)}


def kquant_weights(g: np.random.Generator, fmt: str, n: int, k: int) -> dict:
    """K-quant / IQ4_XS weights in logical form, one super-block of 256
    elements per fp16 scale d (and fp16 dmin for Q4_K / Q5_K):

    * codes uniform over the format's range (Q4_K and IQ4_XS 0..15, Q5_K
      0..31, Q6_K 0..63);
    * d = fp16 of |N(0,1)| * 1e-3 (Q4_K, Q5_K), * 2e-4 (Q6_K), * 1e-4 (IQ4_XS);
      dmin = fp16 of |N(0,1)| * 7.5e-3 (Q4_K, Q5_K);
    * sub-block scales ``sub``: Q4_K / Q5_K / IQ4_XS one 6-bit value (0..63)
      per 32 elements, Q6_K one int8 per 16 elements (uniform -128..127);
      ``mins`` (Q4_K / Q5_K) one 6-bit value per 32 elements.
    """
    assert fmt in KQUANTS and k % KQ_SUPER == 0
    hi = {Q4_K: 16, Q5_K: 32, Q6_K: 64, IQ4_XS: 16}[fmt]
    codes = g.integers(0, hi, size=(n, k), dtype=np.uint8)
    ns = k // KQ_SUPER
    dscale = {Q4_K: 1e-3, Q5_K: 1e-3, Q6_K: 2e-4, IQ4_XS: 1e-4}[fmt]
    w = {"fmt": fmt, "n": n, "k": k, "codes": codes, "d": to_f16_bits(np.abs(g.standard_normal(size=(n, ns))) * dscale)}
    if fmt == Q6_K:
        w["sub"] = g.integers(-128, 128, size=(n, k // 16), dtype=np.int16).astype(np.int8)
    else:
        w["sub"] = g.integers(0, 64, size=(n, k // 32), dtype=np.uint8)
    if fmt in (Q4_K, Q5_K):
        w["dmin"] = to_f16_bits(np.abs(g.standard_normal(size=(n, ns))) * 7.5e-3)
        w["mins"] = g.integers(0, 64, size=(n, k // 32), dtype=np.uint8)
    return w


def q8_0_weights(g: np.random.Generator, n: int, k: int) -> dict:
    assert k % 32 == 0
    codes = g.integers(-127, 128, size=(n, k), dtype=np.int8)
    sc = np.abs(g.standard_normal(size=(n, k // 32))) * 0.02 / 127.0
    return {"fmt": Q8_0, "n": n, "k": k, "codes": codes, "scales": to_f16_bits(sc)}


def q4_0_weights(g: np.random.Generator, n: int, k: int) -> dict:
    assert k % 32 == 0
    codes = g.integers(0, 16, size=(n, k), dtype=np.uint8)
    sc = np.abs(g.standard_normal(size=(n, k // 32))) * 0.01
    return {"fmt": Q4_0, "n": n, "k": k, "codes": codes, "scales": to_f16_bits(sc)}


def x_f32(g: np.random.Generator, m: int, k: int) -> np.ndarray:
    return g.standard_normal(size=(m, k)).astype(np.float32)


def x_bf16(g: np.random.Generator, m: int, k: int) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0,1) draws."""
    return to_bf16_bits(g.standard_normal(size=(m, k)))


def logits_f32(g: np.random.Generator, t: int, e: int) -> np.ndarray:
    return g.standard_normal(size=(t, e)).astype(np.float32)


# --------------------------------------------------------------------------
# the five workloads (full sizes) and scaled-down variants of the same recipe
# --------------------------------------------------------------------------

@dataclass
class DenseQ8:
    """Q8_0 GEMV, fp32 activations."""
    w: dict
    x: np.ndarray  # fp32 [m, k]


def q8_gemv_case(n: int = 1024, k: int = 1024, m: int = 1, seed: int | None = None) -> DenseQ8:
    s = seed_for(1) if seed is None else seed
    w = q8_0_weights(rng(s), n, k)
    x = x_f32(rng(s + 1), m, k)
    return DenseQ8(w=w, x=x)


@dataclass
class DenseNVFP4Layer:
    """Fused gate+up [2I x H] then down [H x I], bf16 activations."""
    gate_up: dict
    down: dict
    x: np.ndarray  # bf16 bits [m, H]


def nvfp4_layer_case(hidden: int = 4096, inter: int = 12288, m: int = 1,
                     seed: int | None = None) -> DenseNVFP4Layer:
    s = seed_for(2) if seed is None else seed
    gu = nvfp4_weights(rng(s), 2 * inter, hidden)
    dn = nvfp4_weights(rng(s + 1), hidden, inter)
    x = x_bf16(rng(s + 2), m, hidden)
    return DenseNVFP4Layer(gate_up=gu, down=dn, x=x)


@dataclass
class W4A8:
    """Q4_0 weights times Q8_0-quantized fp32 activations."""
    w: dict
    x: np.ndarray  # fp32 [m, k]


def w4a8_case(n: int = 17408, k: int = 5120, m: int = 1, seed: int | None = None) -> W4A8:
    s = seed_for(3) if seed is None else seed
    w = q4_0_weights(rng(s), n, k)
    x = x_f32(rng(s + 1), m, k)
    return W4A8(w=w, x=x)


def kquant_case(fmt: str, n: int = 17408, k: int = 5120, m: int = 1, seed: int | None = None) -> W4A8:
    """K-quant / IQ4_XS weights times Q8_0-quantized fp32 activations (the
    27B-class [17408 x 5120] projection by default)."""
    s = seed_for(8, 10 * KQUANTS.index(fmt)) if seed is None else seed
    w = kquant_weights(rng(s), fmt, n, k)
    x = x_f32(rng(s + 1), m, k)
    return W4A8(w=w, x=x)


@dataclass
class MoELayer:
    """Routed experts 0..E-1 plus (optionally) one shared expert stored last."""
    n_experts: int
    top_k: int
    hidden: int
    inter: int
    has_shared: bool
    gate_up: list = field(default_factory=list)  # per expert: nvfp4 dict [2I x H]
    down: list = field(default_factory=list)     # per expert: nvfp4 dict [H x I]
    x: np.ndarray | None = None                  # bf16 bits [t, H]
    logits: np.ndarray | None = None             # fp32 [t, E]


def moe_case(t: int = 1, n_experts: int = 256, top_k: int = 8, hidden: int = 2048,
             inter: int = 512, has_shared: bool = True, seed: int | None = None,
             experts: list | None = None) -> MoELayer:
    """MoE decode workload.

    ``experts`` (optional) lists which expert indices to materialise; the
    others stay ``None`` so that a CPU check can draw just the experts a routing
    selects.  Every expert's weights come from its own seed, so a partial draw
    gives exactly the same bytes as a full one.
    """
    s = seed_for(4) if seed is None else seed
    total = n_experts + (1 if has_shared else 0)
    sel = range(total) if experts is None else experts
    L = MoELayer(n_experts, top_k, hidden, inter, has_shared,
                 gate_up=[None] * total, down=[None] * total)
    for e in sel:
        L.gate_up[e] = nvfp4_weights(rng(s + 10 + 2 * e), 2 * inter, hidden)
        L.down[e] = nvfp4_weights(rng(s + 11 + 2 * e), hidden, inter)
    L.x = x_bf16(rng(s + 1), t, hidden)
    L.logits = logits_f32(rng(s + 2), t, n_experts)
    return L


@dataclass
class Prefill:
    """bf16 X [m, k] times NVFP4 W [n, k]^T, bf16 out."""
    w: dict
    x: np.ndarray  # bf16 bits [m, k]


def prefill_case(m: int = 512, n: int = 12288, k: int = 4096, seed: int | None = None) -> Prefill:
    s = seed_for(5) if seed is None else seed
    w = nvfp4_weights(rng(s), n, k)
    x = x_bf16(rng(s + 1), m, k)
    return Prefill(w=w, x=x)
