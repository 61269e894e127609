"""Planted mistakes in the oracle (on the CPU) must each trip some pin.

Every case below patches one plausible error into the oracle -- a swapped
nibble, a dropped term, a wrong tie rule, a transposed or swapped operand, the
zero activation-scale fault -- and asserts that the pins of tests/pins.py no
longer all pass.  A pin set that let one of these through would not be
pinning the oracle to anything.
"""
import numpy as np
import pytest

import oracle
import pins
from oracle import formats as ofmt
from oracle import moe as omoe
from oracle import nvfp4 as onv
from oracle import routing as ort
from nvfp4_weight_only_moe_amd import workloads as wls


def _tiny():
    wl = wls.WORKLOADS[0]
    ms = [wls.masters(wl, p) for p in (wls.GATE, wls.UP, wls.DOWN)]
    layer = pins._pack_layer(ms)
    _, x = wls.activations(wl)
    ids, w = ort.route_topk(wls.logits(wl), wl.k)
    return ms, layer, x, ids, w


def _all_pins():
    pins.pin_e2m1_table()
    pins.pin_e4m3_decode_vs_torch()
    pins.pin_e4m3_encode_midpoints()
    pins.pin_e2m1_encode_midpoints()
    pins.pin_exact_roundtrip(0)
    pins.pin_nibble_order()
    pins.pin_scale_rule(0)
    pins.pin_zero_and_tiny_tensors()
    lg = np.zeros((2, 8), np.float32)
    lg[1, [1, 4, 6]] = 2.0
    pins.pin_route_bruteforce(lg, 3)
    pins.pin_route_bruteforce(wls.logits(wls.WORKLOADS[0]), 2)
    pins.pin_permutation(np.random.default_rng(0).integers(0, 4, size=(64, 2)), 4)
    pins.pin_textbook_mlp()
    pins.pin_one_hot_columns()
    ms, layer, x, ids, w = _tiny()
    pins.pin_magnitude(x, layer, ids, w, ms)
    pins.pin_bruteforce_layer(x[:3], layer, ids[:3], w[:3])


def test_unmutated_oracle_passes_all_pins():
    _all_pins()


def _swapped_unpack(packed):
    codes = np.empty((packed.shape[0], packed.shape[1] * 2), np.uint8)
    codes[:, 0::2] = packed >> 4
    codes[:, 1::2] = packed & 15
    return codes


def _dequant_without_g(packed, scales, g):
    return _orig_dequant(packed, scales, np.float32(1.0))


_orig_dequant = onv.dequantize


def _e4m3_ties_up(x):
    x = np.asarray(x, np.float64)
    t = ofmt._E4M3_POSITIVE
    hi = np.minimum(np.searchsorted(t, x, side="left"), len(t) - 1)
    lo = np.maximum(hi - 1, 0)
    mid = 0.5 * (t[lo] + t[hi])
    idx = np.where(x >= mid, hi, lo)
    return np.where(x >= t[-1], len(t) - 1, idx).astype(np.uint8)


def _e2m1_ties_down(q):
    q = np.asarray(q, np.float32)
    a = np.abs(q).astype(np.float64)
    t = ofmt.E2M1_MAGNITUDES
    hi = np.minimum(np.searchsorted(t, a, side="left"), len(t) - 1)
    lo = np.maximum(hi - 1, 0)
    mid = 0.5 * (t[lo] + t[hi])
    idx = np.where(a > mid, hi, lo)
    idx = np.where(a >= t[-1], len(t) - 1, idx)
    return (idx | (np.signbit(q).astype(np.int64) << 3)).astype(np.uint8)


def _route_ties_high(logits, k):
    logits = np.asarray(logits, np.float32)
    t, e = logits.shape
    ids = np.empty((t, k), np.int32)
    w = np.empty((t, k))
    for r in range(t):
        order = np.lexsort((-np.arange(e), -logits[r].astype(np.float64)))[:k]
        ids[r] = order
        ex = np.exp(logits[r, order] - logits[r, order].max())
        w[r] = ex / ex.sum()
    return ids, w


def _route_no_renorm(logits, k):
    ids, _ = _orig_route(logits, k)
    lg = np.asarray(logits, np.float64)
    full = np.exp(lg - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    return ids, np.take_along_axis(full, ids.astype(np.int64), axis=1)


_orig_route = ort.route_topk


def _unstable_perm(ids, num_experts):
    c, o, s, p = _orig_perm(ids, num_experts)
    flat = np.asarray(ids).reshape(-1)
    s = np.argsort(-np.arange(flat.size))[np.argsort(flat[::-1], kind="stable")]
    p = np.empty_like(s)
    p[s] = np.arange(flat.size)
    return c, o, s.astype(np.int32), p.astype(np.int32)


_orig_perm = ort.permutation


def _ffn_gate_up_swapped(x, wg, wu, wd, round_h_bf16=False):
    return _orig_ffn(x, wu, wg, wd, round_h_bf16)


def _ffn_sigmoid(x, wg, wu, wd, round_h_bf16=False):
    x = np.asarray(x, np.float64)
    a = x @ np.asarray(wg, np.float64).T
    b = x @ np.asarray(wu, np.float64).T
    return ((1 / (1 + np.exp(-a))) * b) @ np.asarray(wd, np.float64).T


_orig_ffn = omoe.expert_ffn


def _quantize_zero_global(w):
    p, s, g = _orig_quant(w)
    return p, s, np.float32(0.0)


_orig_quant = onv.quantize


def _forward_unweighted(x, layer, ids, weights, tokens=None, round_h_bf16=False):
    return _orig_forward(x, layer, ids, np.ones_like(np.asarray(weights, np.float64)), tokens, round_h_bf16)


_orig_forward = omoe.moe_forward


MUTATIONS = {
    "nibble-order-swapped": [(onv, "unpack_codes", _swapped_unpack)],
    "dequant-drops-global-scale": [(onv, "dequantize", _dequant_without_g),
                                   (omoe, "dequantize", _dequant_without_g)],
    "e4m3-ties-round-up": [(ofmt, "e4m3_encode", _e4m3_ties_up),
                           (oracle, "e4m3_encode", _e4m3_ties_up),
                           (onv, "e4m3_encode", _e4m3_ties_up)],
    "e2m1-ties-round-down": [(ofmt, "e2m1_encode", _e2m1_ties_down),
                             (oracle, "e2m1_encode", _e2m1_ties_down),
                             (onv, "e2m1_encode", _e2m1_ties_down)],
    "route-ties-prefer-high-index": [(ort, "route_topk", _route_ties_high)],
    "route-softmax-not-renormalised": [(ort, "route_topk", _route_no_renorm)],
    "permutation-not-stable": [(ort, "permutation", _unstable_perm)],
    "ffn-gate-and-up-swapped": [(omoe, "expert_ffn", _ffn_gate_up_swapped)],
    "ffn-sigmoid-instead-of-silu": [(omoe, "expert_ffn", _ffn_sigmoid)],
    "zero-global-scale-fault": [(onv, "quantize", _quantize_zero_global)],
    "routing-weights-ignored": [(omoe, "moe_forward", _forward_unweighted)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    for mod, attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, fn)
    with pytest.raises((AssertionError, ValueError)):
        _all_pins()


# ---------------------------------------------------------------- the W4A4 variant
from oracle import w4a4 as ow4  # noqa: E402


def _all_w4a4_pins():
    pins.pin_act_exact_roundtrip(0)
    pins.pin_act_scale_rule(0)
    pins.pin_input_scale_refusal()
    pins.pin_placeholder_underflow()
    pins.pin_w4a4_representable_x()
    pins.pin_w4a4_bruteforce()
    pins.pin_w4a4_magnitude()


_orig_qact = ow4.quantize_activations
_orig_dqact = ow4.dequantize_activations
_orig_fq = ow4.fake_quantize
_orig_ffn4 = ow4.expert_ffn_w4a4


def _qact_scale_ignored(a, input_scale):
    ow4.check_input_scale(input_scale)
    return _orig_qact(a, 1.0)


def _dqact_scale_ignored(packed, scales, input_scale):
    return _orig_dqact(packed, scales, 1.0)


def _dqact_scale_twice(packed, scales, input_scale):
    return (_orig_dqact(packed, scales, input_scale) * np.float32(input_scale)).astype(np.float32)


def _fq_identity(a, input_scale):
    ow4.check_input_scale(input_scale)
    return np.asarray(a, np.float32)


def _ffn4_h_unquantized(xq, wg, wu, wd, input_scale_h, return_h=False):
    x = np.asarray(xq, np.float64)
    a = x @ np.asarray(wg, np.float64).T
    b = x @ np.asarray(wu, np.float64).T
    h = a / (1 + np.exp(-a)) * b
    y = h @ np.asarray(wd, np.float64).T
    return (y, h) if return_h else y


def _ffn4_h_via_bf16(xq, wg, wu, wd, input_scale_h, return_h=False):
    x = np.asarray(xq, np.float64)
    a = x @ np.asarray(wg, np.float64).T
    b = x @ np.asarray(wu, np.float64).T
    h = a / (1 + np.exp(-a)) * b
    hb = omoe._bf16_round(h).astype(np.float32)
    y = _orig_fq(hb, input_scale_h).astype(np.float64) @ np.asarray(wd, np.float64).T
    return (y, h) if return_h else y


def _forward4_h_with_x_scale(x, layer, ids, weights, input_scale_x, input_scale_h, tokens=None):
    return _orig_fwd4(x, layer, ids, weights, input_scale_x, input_scale_x, tokens)


_orig_fwd4 = ow4.moe_forward_w4a4


def _qact_strided_groups(a, input_scale):
    # a reshape-order slip: group j takes k = j, j + K/16, j + 2K/16, ...
    a = np.asarray(a, np.float32)
    k = a.shape[1]
    idx = np.arange(k).reshape(16, k // 16).T.ravel()
    p, s = _orig_qact(np.ascontiguousarray(a[:, idx]), input_scale)
    codes = np.empty((a.shape[0], k), np.uint8)
    codes[:, idx] = onv.unpack_codes(p)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), s


def _check_scale_accepts_anything(s, name="input_scale"):
    return np.float32(1.0 if s is None else s)


W4A4_MUTATIONS = {
    "act-input-scale-ignored": [(ow4, "quantize_activations", _qact_scale_ignored),
                                (ow4, "dequantize_activations", _dqact_scale_ignored)],
    "act-dequant-scale-applied-twice": [(ow4, "dequantize_activations", _dqact_scale_twice)],
    "activations-not-quantized": [(ow4, "fake_quantize", _fq_identity)],
    "h-not-quantized": [(ow4, "expert_ffn_w4a4", _ffn4_h_unquantized)],
    "h-rounded-to-bf16-before-quantization": [(ow4, "expert_ffn_w4a4", _ffn4_h_via_bf16)],
    "h-quantized-with-the-x-scale": [(ow4, "moe_forward_w4a4", _forward4_h_with_x_scale)],
    "act-groups-strided": [(ow4, "quantize_activations", _qact_strided_groups)],
    "zero-input-scale-accepted": [(ow4, "check_input_scale", _check_scale_accepts_anything)],
}


def test_unmutated_w4a4_oracle_passes_all_pins():
    _all_w4a4_pins()


@pytest.mark.parametrize("name", sorted(W4A4_MUTATIONS))
def test_planted_w4a4_mistake_is_caught(name, monkeypatch):
    for mod, attr, fn in W4A4_MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, fn)
    with pytest.raises((AssertionError, ValueError)):
        _all_w4a4_pins()
