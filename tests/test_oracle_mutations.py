"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins
catch every one of them.  This shows the pins are sharp enough to trust."""
import numpy as np
import pytest

import oracle
import synth
from oracle import formats as F
from oracle import ops as O
from tests import test_oracle_a8 as A8
from tests import test_oracle_abs as TA
from tests import test_oracle_fp8 as TF8
from tests import test_oracle_formats as TF
from tests import test_oracle_gemv as TG
from tests import test_oracle_kquants as TK
from tests import test_oracle_moe as TM

pytestmark = pytest.mark.cpu


def _e2m1_wrong_bias(codes):
    c = np.asarray(codes).astype(np.int64)
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e))  # bias dropped
    return np.where(s == 1, -mag, mag)


def _e4m3_fnuz_bias(b):
    b = np.asarray(b).astype(np.int64)
    s, e, m = (b >> 7) & 1, (b >> 3) & 15, b & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    return np.where(s == 1, -mag, mag)


def _nvfp4_divides_tensor_scale(w, rows=None):
    r = O._rows(w, rows)
    c = F.decode_e2m1(w["codes"][r])
    s = F.decode_e4m3(w["scales"][r])
    n, k = c.shape
    return (c.reshape(n, k // 16, 16) * s[:, :, None]).reshape(n, k) / np.float64(np.float32(w["tensor_scale"]))


def _nvfp4_scale_per_32(w, rows=None):
    r = O._rows(w, rows)
    c = F.decode_e2m1(w["codes"][r])
    s = F.decode_e4m3(w["scales"][r])
    n, k = c.shape
    idx = np.minimum(np.arange(k) // 32, s.shape[1] - 1)  # wrong block length
    return c * s[:, idx] * np.float64(np.float32(w["tensor_scale"]))


def _q4_no_offset(w, rows=None):
    r = O._rows(w, rows)
    q = w["codes"][r].astype(np.float64)
    d = F.decode_f16(w["scales"][r])
    n, k = q.shape
    return (q.reshape(n, k // 32, 32) * d[:, :, None]).reshape(n, k)


def _quant_half_away(x):
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    xb = x.reshape(m, k // 32, 32)
    amax = np.max(np.abs(xb), axis=2)
    d32 = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = xb / d32[:, :, None]
    q = np.where(d32[:, :, None] == 0, 0, np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -127, 127)).astype(np.int8)
    return q.reshape(m, k), d32.astype(np.float16).view(np.uint16), q.astype(np.int32).sum(axis=2)


def _router_tie_high(logits, top_k):
    L = np.asarray(logits, dtype=np.float32)
    t, e = L.shape
    ids = np.empty((t, top_k), np.int32)
    w = np.empty((t, top_k))
    for i in range(t):
        order = sorted(range(e), key=lambda j: (-float(L[i, j]), -j))[:top_k]
        ids[i] = order
        ex = np.exp(L[i, order].astype(np.float64) - L[i, order].max())
        w[i] = ex / ex.sum()
    return ids, w


def _swiglu_swapped(h):
    h = np.asarray(h, dtype=np.float64)
    i = h.shape[-1] // 2
    return O.silu(h[..., i:]) * h[..., :i]


def _gemv_transposed_x(w, x, rows=None):
    W = O.dequant(w, rows)
    X = O.act_values(x)
    return X[:, ::-1] @ W.T


def _fp8_tiles(transpose=False, tile=128, columns=True):
    def dq(w, rows=None):
        r = O._rows(w, rows)
        v = F.decode_e4m3(w["codes"][r])
        s = np.asarray(w["scales"], np.float64)
        if not w["tiled"]:
            return v * s.reshape(-1)[0]
        ri = (r // tile)[:, None]
        ci = (np.arange(v.shape[1]) // tile)[None, :] if columns else np.zeros((1, v.shape[1]), np.int64)
        if transpose:
            ri, ci = ci, ri
        ri = np.minimum(ri, s.shape[0] - 1)
        ci = np.minimum(ci, s.shape[1] - 1)
        return v * s[ri, ci]
    return dq


def _kq_min_added(w, rows=None):
    r = O._rows(w, rows)
    q = w["codes"][r].astype(np.float64)
    d = O._per_column(F.decode_f16(w["d"][r]), 256)
    dmin = O._per_column(F.decode_f16(w["dmin"][r]), 256)
    return d * O._per_column(w["sub"][r], 32) * q + dmin * O._per_column(w["mins"][r], 32)


def _kq_fifth_bit_dropped(w, rows=None):
    return ORIG_Q4K(dict(w, codes=w["codes"] & 15), rows)


def _q6k_no_offset(w, rows=None):
    r = O._rows(w, rows)
    d = O._per_column(F.decode_f16(w["d"][r]), 256)
    return d * O._per_column(w["sub"][r].astype(np.int8), 16) * w["codes"][r].astype(np.float64)


def _q6k_sub_blocks_of_32(w, rows=None):
    r = O._rows(w, rows)
    k = w["codes"].shape[1]
    d = O._per_column(F.decode_f16(w["d"][r]), 256)
    sc = O._per_column(w["sub"][r][:, :k // 32].astype(np.int8), 32)
    return d * sc * (w["codes"][r].astype(np.float64) - 32.0)


def _iq4_no_scale_offset(w, rows=None):
    return ORIG_IQ4(dict(w, sub=w["sub"].astype(np.int16) + 32), rows)


def _iq4_codebook_reversed(w, rows=None):
    return ORIG_IQ4(dict(w, codes=15 - w["codes"]), rows)



# ---- tolerance scales (sum |w * x|) and the bf16 output allowance

def _gemv_abs_signed_x(w, x, rows=None):
    return O.act_values(x) @ np.abs(O.dequant(w, rows)).T


def _gemv_abs_after_sum(w, x, rows=None):
    return np.abs(O.act_values(x) @ O.dequant(w, rows).T)


def _gemv_a8_abs_signed_w(w, xq, xd, rows=None):
    return np.abs(O.act_q8_0_values(xq, xd)) @ O.dequant(w, rows).T


def _q4_a8_abs_no_offset(w, xq, xd, rows=None):
    return ORIG_Q4A8ABS(dict(w, codes=w["codes"].astype(np.int64) + 8), xq, xd, rows)


def _moe_gate_up_abs_signed_w(layer, x, csr):
    X = np.abs(O.act_values(x))
    out = np.empty((len(csr["tok"]), 2 * layer.inter))
    for u, e in enumerate(csr["experts"]):
        lo, hi = csr["offsets"][u], csr["offsets"][u + 1]
        out[lo:hi] = X[csr["tok"][lo:hi]] @ O.dequant_nvfp4(layer.gate_up[e]).T
    return out


def _moe_down_abs_signed_a(layer, a, csr, absolute=False):
    if not absolute:
        return ORIG_MOE_DOWN(layer, a, csr)
    A = O.act_values(a)
    out = np.empty((A.shape[0], layer.hidden))
    for u, e in enumerate(csr["experts"]):
        lo, hi = csr["offsets"][u], csr["offsets"][u + 1]
        out[lo:hi] = A[lo:hi] @ np.abs(O.dequant_nvfp4(layer.down[e])).T
    return out


def _prefill_abs_after_sum(w, x, rows=None, cols=None):
    Y, _ = ORIG_PREFILL(w, x, rows, cols)
    return Y, np.abs(Y)


def _bf16_ulp_binade_low(v):
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(v)
    return np.where(v == 0, 2.0 ** -133, np.ldexp(1.0, np.maximum(e - 9, -133)))


ORIG_Q4A8ABS = O.gemv_q4_0_a8_abs
ORIG_MOE_DOWN = O.moe_down
ORIG_PREFILL = O.prefill

ORIG_Q4K = O.dequant_q4_k
ORIG_IQ4 = O.dequant_iq4_xs


def _fp8_pins():
    return [lambda: TF8.test_dequant_matches_torch_decode_and_tile_lookup(300, 384, True),
            TF8.test_gemv_exact_brute_force_across_tiles]


MUTATIONS = [
    ("e2m1 exponent bias dropped", [(F, "decode_e2m1", _e2m1_wrong_bias), (O, "decode_e2m1", _e2m1_wrong_bias),
                                    (oracle, "decode_e2m1", _e2m1_wrong_bias)],
     [TF.test_e2m1_matches_ocp_table, TG.test_ex1_nvfp4_one_block]),
    ("e4m3 read as the FNUZ bias", [(F, "decode_e4m3", _e4m3_fnuz_bias), (O, "decode_e4m3", _e4m3_fnuz_bias),
                                    (oracle, "decode_e4m3", _e4m3_fnuz_bias)],
     [TF.test_e4m3_all_256_against_torch, TG.test_ex6_nvfp4_two_rows_two_blocks_pins_scale_indexing]),
    ("tensor scale divides", [(O, "dequant_nvfp4", _nvfp4_divides_tensor_scale)],
     [TG.test_ex1_nvfp4_one_block]),
    ("NVFP4 block of 32", [(O, "dequant_nvfp4", _nvfp4_scale_per_32)],
     [TG.test_ex6_nvfp4_two_rows_two_blocks_pins_scale_indexing]),
    ("Q4_0 offset of 8 dropped", [(O, "dequant_q4_0", _q4_no_offset)],
     [TG.test_ex3_q4_0_one_block, TG.test_ex8_q4_0_two_rows_two_blocks]),
    ("activations reversed along k", [(O, "gemv", _gemv_transposed_x), (oracle, "gemv", _gemv_transposed_x)],
     [TG.test_nonsquare_orientation, TG.test_ex6_nvfp4_two_rows_two_blocks_pins_scale_indexing]),
    ("quantizer rounds half away from zero", [(O, "quantize_q8_0_act", _quant_half_away),
                                              (oracle, "quantize_q8_0_act", _quant_half_away)],
     [A8.test_quantizer_ties_round_half_even]),
    ("router breaks ties to the higher index", [(O, "route_topk", _router_tie_high),
                                                (oracle, "route_topk", _router_tie_high)],
     [TM.test_ex5_router_tie_to_lower_index]),
    ("gate and up swapped", [(O, "swiglu", _swiglu_swapped), (oracle, "swiglu", _swiglu_swapped)],
     [TM.test_swiglu_gate_is_first_half]),
    ("FP8 scale grid transposed", [(O, "dequant_fp8", _fp8_tiles(transpose=True))], _fp8_pins()),
    ("FP8 tiles of 64", [(O, "dequant_fp8", _fp8_tiles(tile=64))], _fp8_pins()),
    ("FP8 column tiles ignored", [(O, "dequant_fp8", _fp8_tiles(columns=False))], _fp8_pins()),
    ("K-quant min added", [(O, "dequant_q4_k", _kq_min_added)], [TK.test_q4_k_reduces_to_q4_0]),
    ("Q5_K fifth bit dropped", [(O, "dequant_q4_k", _kq_fifth_bit_dropped)], [TK.test_q5_k_uses_the_fifth_bit]),
    ("Q6_K offset of 32 dropped", [(O, "dequant_q6_k", _q6k_no_offset)], [TK.test_q6_k_reduces_to_q8_0]),
    ("Q6_K sub-blocks of 32", [(O, "dequant_q6_k", _q6k_sub_blocks_of_32)],
     [lambda: TK.test_one_hot_sub_block(synth.Q6_K)]),
    ("IQ4_XS scale offset dropped", [(O, "dequant_iq4_xs", _iq4_no_scale_offset)],
     [TK.test_iq4_xs_codebook_and_scale_offset]),
    ("IQ4_XS codebook reversed", [(O, "dequant_iq4_xs", _iq4_codebook_reversed)],
     [TK.test_iq4_xs_codebook_and_scale_offset]),
    ("gemv_abs keeps the activation sign", [(O, "gemv_abs", _gemv_abs_signed_x),
                                            (oracle, "gemv_abs", _gemv_abs_signed_x)],
     [lambda: TA.test_gemv_abs_vs_exact("nvfp4", 3, 32, 2), lambda: TA.test_gemv_abs_vs_exact("q8_0", 4, 64, 2)]),
    ("gemv_abs takes |.| after the sum", [(O, "gemv_abs", _gemv_abs_after_sum),
                                          (oracle, "gemv_abs", _gemv_abs_after_sum)],
     [TA.test_gemv_abs_is_larger_than_the_signed_sum]),
    ("gemv_a8_abs keeps the weight sign", [(O, "gemv_a8_abs", _gemv_a8_abs_signed_w),
                                           (oracle, "gemv_a8_abs", _gemv_a8_abs_signed_w)],
     [lambda: TA.test_gemv_a8_abs_vs_exact(synth.Q4_K)]),
    ("gemv_q4_0_a8_abs drops the offset of 8", [(O, "gemv_q4_0_a8_abs", _q4_a8_abs_no_offset),
                                                (oracle, "gemv_q4_0_a8_abs", _q4_a8_abs_no_offset)],
     [TA.test_gemv_q4_0_a8_abs_vs_exact]),
    ("moe_gate_up_abs keeps the weight sign", [(O, "moe_gate_up_abs", _moe_gate_up_abs_signed_w)],
     [TA.test_moe_gate_up_abs_vs_exact]),
    ("moe_down(absolute) keeps the activation sign", [(O, "moe_down", _moe_down_abs_signed_a)],
     [TA.test_moe_down_abs_vs_exact]),
    ("prefill's abs output takes |.| after the sum", [(O, "prefill", _prefill_abs_after_sum),
                                                      (oracle, "prefill", _prefill_abs_after_sum)],
     [TA.test_prefill_abs_vs_exact]),
    ("bf16_ulp one binade too fine", [(F, "bf16_ulp", _bf16_ulp_binade_low),
                                      (oracle, "bf16_ulp", _bf16_ulp_binade_low)],
     [TA.test_bf16_ulp_vs_torch_spacing]),
]


@pytest.mark.parametrize("name,patches,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, patches, pins, monkeypatch):
    for mod, attr, fn in patches:
        monkeypatch.setattr(mod, attr, fn)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
