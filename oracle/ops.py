"""The block-quantized GEMV path, computed plainly on the CPU in fp64 (test oracle).

Part of the CPU oracle: test infrastructure only, never used by the GPU path.

Weights arrive in the logical form the seeded generators produce: a dict with
``codes`` (one code per element, row-major [n, k]), ``scales`` (raw E4M3 bytes
or fp16 bit patterns, row-major [n, k/B]) and, for NVFP4, ``tensor_scale``.
Activations arrive as fp32 arrays or bf16 bit patterns.  Row ``n`` of a weight
matrix produces output ``y[:, n]``; block ``b`` of row ``n`` covers columns
``[B*b, B*b + B)``.

Every dot product here is the plain definition: dequantize to fp64 (exactly),
then one library matmul in fp64.  Nothing is blocked, fused or reordered beyond
what the definition states.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_bf16, decode_e2m1, decode_e4m3, decode_f16, round_to_bf16

NVFP4_BLOCK = 16
Q_BLOCK = 32


def _rows(w: dict, rows):
    n = w["codes"].shape[0]
    return np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)


# ---------------------------------------------------------------------------
# dequantization (definitions of the three weight formats)
# ---------------------------------------------------------------------------

def dequant_nvfp4(w: dict, rows=None) -> np.ndarray:
    """NVFP4 weight values, exact in fp64.

    value = e2m1(code) * e4m3(block scale) * tensor scale, one E4M3 scale per
    16 consecutive elements of a row (NVFP4: LumenLLM README, feature list
    "Quantization"; bw24 README, "NVFP4 (W4) decode path").  The tensor scale
    multiplies (the plain reading of a per-tensor fp32 scale).  e2m1*e4m3 has at
    most 6 significant bits and the tensor scale 24, so the fp64 product is exact.
    """
    r = _rows(w, rows)
    c = decode_e2m1(w["codes"][r])
    s = decode_e4m3(w["scales"][r])
    n, k = c.shape
    blk = c.reshape(n, k // NVFP4_BLOCK, NVFP4_BLOCK) * s[:, :, None]
    return blk.reshape(n, k) * np.float64(np.float32(w["tensor_scale"]))


def dequant_nvfp4_f32(w: dict, rows=None) -> np.ndarray:
    """NVFP4 weights rounded once to fp32 (round to nearest even)."""
    return dequant_nvfp4(w, rows).astype(np.float32)


def dequant_q8_0(w: dict, rows=None) -> np.ndarray:
    """Q8_0 weight values: fp16 scale d per 32 elements times the int8 code.

    (Q8_0: memra README, "Decode kernels" and its model table; Lumen page,
    "Format" section.)  Exact in fp64 and in fp32 (at most 19 significant bits).
    """
    r = _rows(w, rows)
    q = w["codes"][r].astype(np.float64)
    d = decode_f16(w["scales"][r])
    n, k = q.shape
    return (q.reshape(n, k // Q_BLOCK, Q_BLOCK) * d[:, :, None]).reshape(n, k)


def dequant_q4_0(w: dict, rows=None) -> np.ndarray:
    """Q4_0 weight values: fp16 scale d per 32 elements times (code - 8).

    (Q4_0: memra README, "Decode kernels" and its Gemma rows; Lumen page,
    "Format" section.)  Exact in fp64 and fp32.
    """
    r = _rows(w, rows)
    q = w["codes"][r].astype(np.float64) - 8.0
    d = decode_f16(w["scales"][r])
    n, k = q.shape
    return (q.reshape(n, k // Q_BLOCK, Q_BLOCK) * d[:, :, None]).reshape(n, k)


FP8_TILE = 128


def dequant_fp8(w: dict, rows=None) -> np.ndarray:
    """FP8 weight values: e4m3(code) times an fp32 scale, exact in fp64.

    E4M3 weights (LumenLLM README, feature list "Quantization": native FP8
    (E4M3); model table: its 9B model runs FP8).  Scales: one per tensor, or
    one per 128 x 128 tile of W when ``w["tiled"]`` (the block-128 FP8
    checkpoints of the memra README, feature list "Loaders"); tile (i, j)
    scales rows [128 i, 128 i + 128) and columns [128 j, 128 j + 128).
    """
    r = _rows(w, rows)
    v = decode_e4m3(w["codes"][r])
    s = np.asarray(w["scales"], dtype=np.float32).astype(np.float64)
    if not w["tiled"]:
        return v * s.reshape(-1)[0]
    k = v.shape[1]
    cols = np.arange(k) // FP8_TILE
    return v * s[(r // FP8_TILE)[:, None], cols[None, :]]


# ---------------------------------------------------------------------------
# K-quants and IQ4_XS (super-blocks of 256 elements)
#
# The pages name these formats without defining them: K-quant split-plane
# matvecs (memra README, feature list "Decode kernels"), GGUF models in
# Q4_K / Q5_K / Q6_K and a 35B MoE in IQ4_XS (bw24 README, requirements and
# model list; memra README, model table).  The definitions below are the
# public GGUF ones, stated on the logical values (codes and scales), not on
# GGUF's byte packing:
#
# * Q4_K / Q5_K: per 256 elements an fp16 scale d and an fp16 scale dmin; per
#   32-element sub-block j a 6-bit scale sc_j and a 6-bit min m_j; 4-bit
#   (Q4_K) or 5-bit (Q5_K) codes q:  w = d * sc_j * q - dmin * m_j.
# * Q6_K: per 256 elements an fp16 scale d; per 16-element sub-block j an
#   int8 scale sc_j; 6-bit codes q:  w = d * sc_j * (q - 32).
# * IQ4_XS: per 256 elements an fp16 scale d; per 32-element sub-block j a
#   6-bit scale ls_j; 4-bit indices q into the fixed non-linear 16-entry
#   codebook T (the IQ4_NL values):  w = d * (ls_j - 32) * T[q].
# ---------------------------------------------------------------------------

KQ_SUPER = 256
IQ4_NL_VALUES = np.array([-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113],
                         dtype=np.float64)


def _per_column(v: np.ndarray, width: int) -> np.ndarray:
    """Spread per-(sub-)block values over the columns they scale."""
    return np.repeat(np.asarray(v, dtype=np.float64), width, axis=1)


def dequant_q4_k(w: dict, rows=None) -> np.ndarray:
    """Q4_K / Q5_K values d*sc_j*q - dmin*m_j (same rule; Q5_K codes go to 31).

    Each product is exact in fp64 (at most 22 significant bits); the
    difference is exact whenever d and dmin lie within 2^30 of each other,
    which every realistic scale pair (and every generated one) does.
    """
    r = _rows(w, rows)
    q = w["codes"][r].astype(np.float64)
    d = _per_column(decode_f16(w["d"][r]), KQ_SUPER)
    dmin = _per_column(decode_f16(w["dmin"][r]), KQ_SUPER)
    sc = _per_column(w["sub"][r], 32)
    mn = _per_column(w["mins"][r], 32)
    return d * sc * q - dmin * mn


def dequant_q6_k(w: dict, rows=None) -> np.ndarray:
    """Q6_K values d*sc_j*(q - 32), sc_j int8 per 16 elements (exact: <= 24 bits)."""
    r = _rows(w, rows)
    q = w["codes"][r].astype(np.float64) - 32.0
    d = _per_column(decode_f16(w["d"][r]), KQ_SUPER)
    sc = _per_column(w["sub"][r].astype(np.int8), 16)
    return d * sc * q


def dequant_iq4_xs(w: dict, rows=None) -> np.ndarray:
    """IQ4_XS values d*(ls_j - 32)*T[q] (exact: <= 24 significant bits)."""
    r = _rows(w, rows)
    t = IQ4_NL_VALUES[w["codes"][r]]
    d = _per_column(decode_f16(w["d"][r]), KQ_SUPER)
    ls = _per_column(w["sub"][r], 32) - 32.0
    return d * ls * t


def dequant(w: dict, rows=None) -> np.ndarray:
    f = {"nvfp4": dequant_nvfp4, "q8_0": dequant_q8_0, "q4_0": dequant_q4_0, "fp8": dequant_fp8,
         "q4_k": dequant_q4_k, "q5_k": dequant_q4_k, "q6_k": dequant_q6_k, "iq4_xs": dequant_iq4_xs}[w["fmt"]]
    return f(w, rows)


def act_values(x) -> np.ndarray:
    """Activation values in fp64: bf16 bit patterns (uint16) or fp32 arrays."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# fused-dequant GEMV y = W x (per token), and the tolerance it is held to
# ---------------------------------------------------------------------------

def gemv(w: dict, x, rows=None) -> np.ndarray:
    """y[m, n] = sum_k w[n, k] * x[m, k] with exactly dequantized w, in fp64.

    The decode step's matrix-vector product over block-quantized weights
    (LumenLLM README, "Kernels": warp-shuffle GEMVs; bw24 README, "NVFP4 (W4)
    decode path"; memra README, "Decode kernels": split-plane matvecs).
    ``x`` is [m, k] (fp32, or bf16 bit patterns).  Returns [m, len(rows)].
    """
    W = dequant(w, rows)
    X = act_values(x)
    return X @ W.T


def gemv_abs(w: dict, x, rows=None) -> np.ndarray:
    """sum_k |w[n, k] * x[m, k]|, the scale of the rounding error of y[m, n]."""
    W = np.abs(dequant(w, rows))
    X = np.abs(act_values(x))
    return X @ W.T


def tolerance(abs_sum) -> np.ndarray:
    """Allowed |y_gpu - y_ref| per output: 1e-5 * sum|w*x| + 1e-6."""
    return 1e-5 * np.asarray(abs_sum, dtype=np.float64) + 1e-6


# ---------------------------------------------------------------------------
# W4A8: Q8_0-quantized activations and the integer block dot
# ---------------------------------------------------------------------------

def quantize_q8_0_act(x):
    """Quantize fp32 activations to Q8_0 (int8 codes + fp16 scale per 32).

    The W4A8 path (bw24 README, "NVFP4 (W4) decode path": dp4a matvec and the
    int8 W4A8 GEMM) needs int8 activations; the pages do not say how they are
    made.  Reading taken (the plain Q8_0 recipe, with every rounding stated):

    * amax = max |x| over the 32-element block (exact in fp32);
    * d32 = amax / 127 as a correctly rounded fp32 division;
    * d16 = d32 rounded to fp16 (nearest even) -- the scale that is stored and
      that the dot product uses;
    * q = clamp(round_half_even(x / d32), -127, 127), with x / d32 a correctly
      rounded fp32 division (numpy's float32 division is IEEE);
    * a block with amax = 0 gets d = 0 and q = 0;
    * xs = sum of q over the block (int32), used to fold the Q4_0 offset of 8
      out of the integer dot.

    Returns (xq int8 [m, k], xd fp16 bits uint16 [m, k/32], xs int32 [m, k/32]).
    """
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    xb = x.reshape(m, k // Q_BLOCK, Q_BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    d32 = (amax / np.float32(127.0)).astype(np.float32)
    d16 = d32.astype(np.float16)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (xb / d32[:, :, None]).astype(np.float32)
    q = np.where(d32[:, :, None] == 0, np.float32(0), np.clip(np.rint(ratio), -127, 127))
    q = q.astype(np.int8)
    xs = q.astype(np.int32).sum(axis=2, dtype=np.int32)
    return q.reshape(m, k), d16.view(np.uint16), xs


def block_isums_q4_0_a8(w: dict, xq, rows=None) -> np.ndarray:
    """isum[m, n, b] = sum_{j in block b} (q_w[n, j] - 8) * q_x[m, j], exact int64.

    The integer block dot of the W4A8 path (bw24 README: dp4a, "W4A8").
    """
    r = _rows(w, rows)
    qw = w["codes"][r].astype(np.int64) - 8
    qx = np.asarray(xq).astype(np.int64)
    n, k = qw.shape
    m = qx.shape[0]
    nb = k // Q_BLOCK
    return np.einsum("nbj,mbj->mnb", qw.reshape(n, nb, Q_BLOCK), qx.reshape(m, nb, Q_BLOCK))


def gemv_q4_0_a8(w: dict, xq, xd, rows=None) -> np.ndarray:
    """y[m, n] = sum_b d_w[n, b] * d_x[m, b] * isum[m, n, b], in fp64."""
    r = _rows(w, rows)
    isum = block_isums_q4_0_a8(w, xq, r).astype(np.float64)
    dw = decode_f16(w["scales"][r])          # [n, nb]
    dx = decode_f16(np.asarray(xd))          # [m, nb]
    return np.einsum("mnb,nb,mb->mn", isum, dw, dx)


def gemv_q4_0_a8_abs(w: dict, xq, xd, rows=None) -> np.ndarray:
    """sum_k |w_k * xhat_k| with xhat = d_x * q_x (the dequantized activation)."""
    r = _rows(w, rows)
    qw = np.abs(w["codes"][r].astype(np.int64) - 8)
    qx = np.abs(np.asarray(xq).astype(np.int64))
    n, k = qw.shape
    m = qx.shape[0]
    nb = k // Q_BLOCK
    s = np.einsum("nbj,mbj->mnb", qw.reshape(n, nb, Q_BLOCK), qx.reshape(m, nb, Q_BLOCK))
    dw = np.abs(decode_f16(w["scales"][r]))
    dx = np.abs(decode_f16(np.asarray(xd)))
    return np.einsum("mnb,nb,mb->mn", s.astype(np.float64), dw, dx)


def act_q8_0_values(xq, xd) -> np.ndarray:
    """The dequantized Q8_0 activation x_hat = d_x * q_x, exact in fp64."""
    qx = np.asarray(xq).astype(np.float64)
    m, k = qx.shape
    return qx * _per_column(decode_f16(np.asarray(xd)), Q_BLOCK)


def gemv_a8(w: dict, xq, xd, rows=None) -> np.ndarray:
    """y[m, n] = sum_k w[n, k] * x_hat[m, k] with x_hat the Q8_0 activation.

    The K-quant and IQ4_XS matvecs take Q8_0 activations, as the W4A8 path
    does (memra README, "Decode kernels": K-quant split-plane matvecs with
    warp-level dp4a, an int8 dot that needs int8 activations).  Plain
    definition: both operands dequantized exactly, one fp64 matmul.
    """
    return act_q8_0_values(xq, xd) @ dequant(w, rows).T


def gemv_a8_abs(w: dict, xq, xd, rows=None) -> np.ndarray:
    """sum_k |w[n, k] * x_hat[m, k]|, the scale of the rounding error."""
    return np.abs(act_q8_0_values(xq, xd)) @ np.abs(dequant(w, rows)).T


# ---------------------------------------------------------------------------
# MoE: router, expert-major grouping, SwiGLU, combine
# ---------------------------------------------------------------------------

def route_topk(logits, top_k: int):
    """Top-k experts per token and their renormalised softmax weights.

    Softmax top-k routing is implied by the MoE models the pages run (bw24
    README, "Sigmoid-router MoE" contrasts its sigmoid router with it and notes
    that top-k routing is discontinuous, so selection must be exact).  Reading
    taken: select the k largest fp32 logits (ties go to the lower expert index;
    this picks the same set as the k largest softmax probabilities), order them
    by logit descending then index ascending, weight = exp(l - l_max) / sum of
    exp(l - l_max) over the selected k (= the global softmax renormalised over
    the selection).  Returns (ids int32 [t, k], weights fp64 [t, k]).
    """
    L = np.asarray(logits, dtype=np.float32)
    t, e = L.shape
    ids = np.empty((t, top_k), dtype=np.int32)
    wts = np.empty((t, top_k), dtype=np.float64)
    for i in range(t):
        order = sorted(range(e), key=lambda j: (-float(L[i, j]), j))[:top_k]
        ids[i] = order
        sel = L[i, order].astype(np.float64)
        ex = np.exp(sel - sel.max())
        wts[i] = ex / ex.sum()
    return ids, wts


def group_by_expert(ids, n_experts: int, has_shared: bool) -> dict:
    """Expert-major CSR of the routed (token, slot) pairs.

    bw24 README, feature list "MoE on 24 GB": expert-major CSR batching, so that
    each active expert's weights are read once for all the tokens routed to it.
    Convention (the pages give none): active experts in ascending id, then the
    shared expert (id = n_experts) holding every token with slot = top_k; inside
    one expert, pairs in ascending (token, slot).

    Returns dict(experts [U], offsets [U+1], tok [P], slot [P]) as int32.
    """
    ids = np.asarray(ids, dtype=np.int64)
    t, k = ids.shape
    experts, offsets, tok, slot = [], [0], [], []
    for e in sorted(set(ids.ravel().tolist())):
        experts.append(e)
        for i in range(t):
            for s in range(k):
                if ids[i, s] == e:
                    tok.append(i)
                    slot.append(s)
        offsets.append(len(tok))
    if has_shared:
        experts.append(n_experts)
        for i in range(t):
            tok.append(i)
            slot.append(k)
        offsets.append(len(tok))
    as32 = lambda a: np.asarray(a, dtype=np.int32)  # noqa: E731
    return {"experts": as32(experts), "offsets": as32(offsets), "tok": as32(tok), "slot": as32(slot)}


def silu(g) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g))."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(h) -> np.ndarray:
    """a = silu(g) * u with g = h[:, :I] and u = h[:, I:] (fp64).

    The MLP activation between the fused gate/up and the down projection of the
    dense and MoE MLPs the pages run (LumenLLM README, model list: dense MLP /
    MoE).  Reading taken: the fused matrix's first I rows are the gate, the next
    I rows the up projection.
    """
    h = np.asarray(h, dtype=np.float64)
    i = h.shape[-1] // 2
    return silu(h[..., :i]) * h[..., i:]


def swiglu_bf16(h) -> np.ndarray:
    """SwiGLU output rounded once to bf16 (the down projection's input dtype)."""
    return round_to_bf16(swiglu(h))


def moe_gate_up(layer, x, csr: dict) -> np.ndarray:
    """h[p] = W_gate_up[expert of pair p] . x[token of pair p], fp64 [P, 2I]."""
    X = act_values(x)
    P = len(csr["tok"])
    out = np.empty((P, 2 * layer.inter))
    for u, e in enumerate(csr["experts"]):
        lo, hi = csr["offsets"][u], csr["offsets"][u + 1]
        W = dequant_nvfp4(layer.gate_up[e])
        out[lo:hi] = X[csr["tok"][lo:hi]] @ W.T
    return out


def moe_gate_up_abs(layer, x, csr: dict) -> np.ndarray:
    X = np.abs(act_values(x))
    P = len(csr["tok"])
    out = np.empty((P, 2 * layer.inter))
    for u, e in enumerate(csr["experts"]):
        lo, hi = csr["offsets"][u], csr["offsets"][u + 1]
        W = np.abs(dequant_nvfp4(layer.gate_up[e]))
        out[lo:hi] = X[csr["tok"][lo:hi]] @ W.T
    return out


def moe_down(layer, a, csr: dict, absolute: bool = False) -> np.ndarray:
    """o[p] = W_down[expert of pair p] . a[p], fp64 [P, H]; ``a`` in CSR pair order."""
    A = act_values(a)
    if absolute:
        A = np.abs(A)
    P = A.shape[0]
    out = np.empty((P, layer.hidden))
    for u, e in enumerate(csr["experts"]):
        lo, hi = csr["offsets"][u], csr["offsets"][u + 1]
        W = dequant_nvfp4(layer.down[e])
        if absolute:
            W = np.abs(W)
        out[lo:hi] = A[lo:hi] @ W.T
    return out


def moe_combine(o, weights, csr: dict, t: int, top_k: int) -> np.ndarray:
    """y[t] = sum_s w[t, s] * o[pair (t, s)] + o[pair (t, shared)], fp64 [T, H].

    Weighted sum of the routed experts' outputs plus the shared expert's output
    with unit weight (reading taken: the pages give no shared-expert gate).
    """
    o = np.asarray(o, dtype=np.float64)
    W = np.asarray(weights, dtype=np.float64)
    y = np.zeros((t, o.shape[1]))
    for p in range(len(csr["tok"])):
        ti, s = int(csr["tok"][p]), int(csr["slot"][p])
        y[ti] += (W[ti, s] if s < top_k else 1.0) * o[p]
    return y


def moe_forward(layer, x, ids, weights) -> dict:
    """The whole MoE decode layer in fp64 from the original x (chained oracle)."""
    csr = group_by_expert(ids, layer.n_experts, layer.has_shared)
    h = moe_gate_up(layer, x, csr)
    a = swiglu(h)
    o = moe_down(layer, a, csr)
    y = moe_combine(o, weights, csr, np.asarray(x).shape[0], layer.top_k)
    return {"csr": csr, "h": h, "a": a, "o": o, "y": y}


# ---------------------------------------------------------------------------
# small-M prefill GEMM
# ---------------------------------------------------------------------------

def prefill(w: dict, x, rows=None, cols=None):
    """Y[m, n] = s_t * sum_k D[n, k] * X[m, k], with D = e2m1 * e4m3 exactly.

    The prefill-side GEMM over the same NVFP4 weights (LumenLLM README,
    "Kernels": NVFP4 grouped-MoE prefill and tensor-core GEMMs; memra README,
    known gaps: prefill kept at bf16-activation numerics, not W4A4).  ``rows``
    selects tokens (rows of X), ``cols`` selects weight rows.  Returns
    (Y fp64, sum |s_t * D * X| fp64), both [len(rows), len(cols)].
    """
    X = act_values(x)
    if rows is not None:
        X = X[np.asarray(rows)]
    W = dequant_nvfp4(w, cols)
    return X @ W.T, np.abs(X) @ np.abs(W).T
