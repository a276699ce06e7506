"""Scalar number formats, decoded from their bit fields in fp64 (test oracle).

Part of the CPU oracle: test infrastructure only, never used by the GPU path.

Each decoder works from the public bit-field definition of its format, not from
a table copied out of a kernel:

* E2M1 (4-bit float, OCP Microscaling Formats v1.0): sign s = bit 3, exponent
  e = bits 2..1 (bias 1), mantissa m = bit 0.  e = 0 is subnormal (m * 0.5);
  otherwise (1 + m/2) * 2**(e-1).  No infinities or NaN; code 8 is -0.
* E4M3 (OCP 8-bit Floating Point v1.0, the "FN" variant without infinities):
  s = bit 7, e = bits 6..3 (bias 7), m = bits 2..0.  e = 15 with m = 7 is NaN;
  e = 0 is subnormal (m/8) * 2**-6; otherwise (1 + m/8) * 2**(e-7).
* binary16 (IEEE 754): s = bit 15, e = bits 14..10 (bias 15), m = bits 9..0.
* bfloat16: the upper 16 bits of an IEEE binary32 (s, 8-bit e bias 127, 7-bit m).

These are the scale and code formats of NVFP4 (LumenLLM README, feature list
"Quantization"; bw24 README, "NVFP4 (W4) decode path") and of Q8_0 / Q4_0
(memra README, "Decode kernels"; Lumen page, "Format" section).  The pages do
not spell the bit fields out; the OCP / IEEE definitions are the plain reading.
"""
from __future__ import annotations

import numpy as np


def decode_e2m1(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_e4m3(b) -> np.ndarray:
    b = np.asarray(b).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    sub = (m / 8.0) * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where(e == 0, sub, nor)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_f16(bits) -> np.ndarray:
    u = np.asarray(bits).astype(np.int64) & 0xFFFF
    s = (u >> 15) & 1
    e = (u >> 10) & 31
    m = u & 1023
    sub = (m / 1024.0) * 2.0 ** -14
    nor = (1.0 + m / 1024.0) * np.exp2(e - 15.0)
    mag = np.where(e == 0, sub, nor)
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_bf16(bits) -> np.ndarray:
    u = np.asarray(bits).astype(np.int64) & 0xFFFF
    s = (u >> 15) & 1
    e = (u >> 7) & 255
    m = u & 127
    sub = (m / 128.0) * 2.0 ** -126
    nor = (1.0 + m / 128.0) * np.exp2(e - 127.0)
    mag = np.where(e == 0, sub, nor)
    mag = np.where(e == 255, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of fp64 values, rounded once.

    Rounds the fp64 value directly to 8 significant bits (no intermediate fp32
    rounding, which could round twice).  Below 2**-126 the bf16 grid is the
    fixed subnormal step 2**-133.  Values beyond the largest finite bf16 round to
    infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    fin = np.isfinite(v)
    out[~fin] = v[~fin]
    a = v[fin]
    _, e = np.frexp(a)  # a = f * 2**e, 0.5 <= |f| < 1
    # exponent of the grid step: 8 significant bits in the binade of a,
    # never finer than the subnormal step.
    step_exp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(a, -step_exp))  # exact scaling, then ties-to-even
    r = np.ldexp(q, step_exp)
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > max_bf16, np.sign(a) * np.inf, r)
    out[fin] = r
    return out


def bf16_ulp(v) -> np.ndarray:
    """Spacing of the bf16 grid at |v| (2**(e-8) with |v| in [2**(e-1), 2**e))."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(v)
    return np.where(v == 0, 2.0 ** -133, np.ldexp(1.0, np.maximum(e - 8, -133)))


def f32_bits(v) -> np.ndarray:
    """IEEE binary32 bit patterns (uint32) of values already in fp32."""
    return np.asarray(v, dtype=np.float32).view(np.uint32)
