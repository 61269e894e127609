"""Checks that pin the oracle to facts outside itself.

Each function raises AssertionError when the oracle disagrees with a closed
form, a library routine, brute force or an invariant.  The pin tests call them
on the real oracle; tests/test_oracle_mutations.py plants plausible mistakes
in the oracle (on the CPU) and shows that some pin catches each one.
"""

import math

import numpy as np
import torch

import oracle
from oracle import nvfp4 as onv
from oracle import routing as ort
from oracle import moe as omoe

# Value table of FP4 E2M1 written out from the format definition (OCP
# Microscaling Formats v1.0): magnitudes of codes 0..7.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ---------------------------------------------------------------- formats
def pin_e2m1_table():
    vals = oracle.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == E2M1_TABLE
    assert list(-vals[8:]) == E2M1_TABLE
    assert np.all(np.signbit(vals[8:])) and not np.any(np.signbit(vals[:8]))
    # ordering: magnitudes strictly increase with the code
    assert np.all(np.diff(vals[:8]) > 0)


def pin_e4m3_decode_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.e4m3_decode(np.arange(256))
    nan_ref, nan_mine = np.isnan(ref), np.isnan(mine)
    assert np.array_equal(nan_ref, nan_mine)
    assert np.array_equal(ref[~nan_ref], mine[~nan_mine])
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(mine[~nan_mine]))


def pin_e4m3_encode_midpoints():
    vals = oracle.e4m3_decode(np.arange(0x7F))
    # every finite non-negative value encodes to itself
    assert np.array_equal(oracle.e4m3_encode(vals.astype(np.float32)), np.arange(0x7F))
    for i in range(0x7E):
        mid = np.float32((vals[i] + vals[i + 1]) / 2)
        assert float(mid) == (vals[i] + vals[i + 1]) / 2          # exact in fp32
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        even = i if i % 2 == 0 else i + 1
        got = oracle.e4m3_encode(np.array([below, mid, above], dtype=np.float32))
        assert list(got) == [i, even, i + 1], (i, got)
    # saturation instead of NaN
    assert list(oracle.e4m3_encode(np.array([448, 460, 464, 1e30], np.float32))) == [0x7E] * 4
    # below half of the smallest subnormal flushes to zero; exactly half ties to 0
    assert list(oracle.e4m3_encode(np.array([2.0 ** -11, 2.0 ** -10], np.float32))) == [0, 0]


def pin_e4m3_encode_vs_torch(seed=0, n=200_000):
    g = np.random.default_rng(seed)
    x = np.concatenate([
        g.uniform(0, 464, n).astype(np.float32),
        np.exp(g.uniform(np.log(1e-12), np.log(463.0), n)).astype(np.float32),
    ])
    x = x[x < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


def pin_e2m1_encode_midpoints():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want_tie = [0, 2, 2, 4, 4, 6, 6]            # the even code of each pair
    for i, (m, t) in enumerate(zip(mids, want_tie)):
        m32 = np.float32(m)
        below = np.nextafter(m32, np.float32(0))
        above = np.nextafter(m32, np.float32(np.inf))
        got = oracle.e2m1_encode(np.array([below, m32, above], np.float32))
        assert list(got) == [i, t, i + 1], (m, got)
        neg = oracle.e2m1_encode(np.array([-below, -m32, -above], np.float32))
        assert list(neg) == [8 + i, 8 + t, 8 + i + 1], (m, neg)
    assert list(oracle.e2m1_encode(np.array([6.0, 6.4, 1e9, -7.0], np.float32))) == [7, 7, 7, 15]
    assert list(oracle.e2m1_encode(np.array([0.0, -0.0, -0.1, 0.1], np.float32))) == [0, 8, 8, 0]
    # every table value encodes to itself
    assert list(oracle.e2m1_encode(np.array(E2M1_TABLE, np.float32))) == list(range(8))


# ---------------------------------------------------------------- quantization
def representable_tensor(seed, n=24, k=96):
    """A tensor whose every element is exactly c * s * g, with g = 2**-12,
    scales drawn from the E4M3 set, a +-6 code in every group and one group
    at s = 448 -- so quantization must give back codes, scales and g exactly.
    Returns (W, codes [n, k], scale bytes [n, k/16], g)."""
    g = np.float32(2.0 ** -12)
    r = np.random.default_rng(seed)
    codes = r.integers(0, 16, size=(n, k)).astype(np.uint8)
    sb = r.integers(1, 0x7F, size=(n, k // 16)).astype(np.uint8)   # 0x01..0x7E
    sb[0, 0] = 0x7E
    for i in range(n):
        for j in range(k // 16):
            codes[i, 16 * j + r.integers(0, 16)] = 7 if r.random() < 0.5 else 15
    c = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6],
                 dtype=np.float32)[codes]
    s = torch.from_numpy(sb).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    w = (c * np.repeat(s, 16, axis=1)).astype(np.float32) * g
    return w.astype(np.float32), codes, sb, g


def pin_exact_roundtrip(seed=0):
    w, codes, sb, g = representable_tensor(seed)
    packed, scales, g2 = onv.quantize(w)
    assert g2 == g
    assert np.array_equal(scales, sb)
    assert np.array_equal(onv.unpack_codes(packed), codes)
    back = onv.dequantize(packed, scales, g2)
    assert np.array_equal(back.view(np.uint32), w.view(np.uint32))


def pin_nibble_order():
    w = np.zeros((2, 32), np.float32)
    w[0, 0] = 1.0      # even k -> low nibble of byte 0
    w[1, 3] = -1.0     # odd k -> high nibble of byte 1
    packed, scales, g = onv.quantize(w)
    assert packed[0, 0] == 0x07 and packed[0, 1] == 0x00
    assert packed[1, 1] == 0xF0 and packed[1, 0] == 0x00
    assert abs(g - 1.0 / 2688) < 1e-12


def pin_scale_rule(seed=0):
    """Group scales and the global scale against torch's own E4M3 conversion
    and the plain quotient; codes against a brute-force nearest search."""
    r = np.random.default_rng(seed)
    w = (0.02 * r.standard_normal((16, 128))).astype(np.float32)
    w[3, :16] = 0.0                                   # an all-zero group
    packed, scales, g = onv.quantize(w)
    amax = np.float32(np.max(np.abs(w)))
    assert g == np.float32(amax / np.float32(2688.0))
    amax_g = np.abs(w).reshape(16, 8, 16).max(axis=2)
    s_f = (amax_g / np.float32(6)) / g
    ref = torch.from_numpy(s_f.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, ref)
    s_q = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    codes = onv.unpack_codes(packed)
    mags = np.array(E2M1_TABLE)
    for i in range(16):
        for j in range(128):
            d = np.float32(s_q[i, j // 16] * g)
            if d == 0:
                assert codes[i, j] & 7 == 0
                continue
            q = float(np.float32(w[i, j] / d))
            dist = np.abs(abs(q) - mags)
            best = np.flatnonzero(dist == dist.min())
            want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            assert codes[i, j] & 7 == want, (i, j, q, codes[i, j])
            assert (codes[i, j] >> 3) == int(np.signbit(np.float32(q)))


def pin_zero_and_tiny_tensors():
    z = np.zeros((4, 32), np.float32)
    p, s, g = onv.quantize(z)
    assert g == np.float32(1.0) and not p.any() and not s.any()
    zn = -np.zeros((4, 32), np.float32)
    p, s, g = onv.quantize(zn)
    assert np.all(p == 0x88) and g == np.float32(1.0)
    tiny = np.zeros((2, 32), np.float32)
    tiny[0, 5] = np.float32(1e-44)          # amax / 2688 underflows to 0
    tiny[1, 7] = np.float32(-1e-45)
    p, s, g = onv.quantize(tiny)
    assert g == np.float32(1.0) and not s.any()
    codes = onv.unpack_codes(p)
    assert codes[0, 5] == 0 and codes[1, 7] == 8


def pin_roundtrip_cosine_band(seed=0):
    """Gaussian N(0, 0.02) masters: weight round-trip cosine in a soft band.
    The pages report 0.99665 for real weights ("GLM-5.3-Flash on Blackwell",
    "The quantization"); Gaussian weights land near 0.995."""
    r = np.random.default_rng(seed)
    w = (0.02 * r.standard_normal((256, 1024))).astype(np.float32)
    back = onv.dequantize(*onv.quantize(w)).astype(np.float64)
    w64 = w.astype(np.float64)
    cos = float((w64 * back).sum() / np.linalg.norm(w64) / np.linalg.norm(back))
    assert 0.99 <= cos <= 0.999, cos
    ratio = float(np.linalg.norm(back) / np.linalg.norm(w64))
    assert 0.95 <= ratio <= 1.05, ratio
    return cos


# ---------------------------------------------------------------- routing
def pin_route_bruteforce(logits, k):
    ids, w = ort.route_topk(logits, k)
    t, e = logits.shape
    for row in range(t):
        order = sorted(range(e), key=lambda i: (-float(logits[row, i]), i))[:k]
        assert list(ids[row]) == order, (row, list(ids[row]), order)
        sel = [float(logits[row, i]) for i in order]
        m = max(sel)
        ex = [math.exp(v - m) for v in sel]
        s = math.fsum(ex)
        assert np.allclose(w[row], [v / s for v in ex], rtol=1e-13, atol=0)
        # softmax over all E, then renormalised over the selected k
        full = np.exp(logits[row].astype(np.float64) - logits[row].max())
        full /= full.sum()
        ren = full[order] / full[order].sum()
        assert np.allclose(w[row], ren, rtol=1e-12, atol=1e-15)
        assert abs(math.fsum(w[row]) - 1.0) <= 1e-12


def pin_permutation(ids, E):
    counts, offsets, sorted_slots, slot_pos = ort.permutation(ids, E)
    flat = np.asarray(ids).reshape(-1)
    want = sorted(range(flat.size), key=lambda i: (int(flat[i]), i))
    assert list(sorted_slots) == want
    assert sorted(sorted_slots.tolist()) == list(range(flat.size))
    assert np.array_equal(slot_pos[sorted_slots], np.arange(flat.size))
    assert counts.sum() == flat.size and offsets[0] == 0 and offsets[-1] == flat.size
    assert np.all(np.diff(offsets) == counts)
    for e in range(E):
        seg = flat[sorted_slots[offsets[e]:offsets[e + 1]]]
        assert np.all(seg == e)


# ---------------------------------------------------------------- FFN / layer
def _pack_layer(ms):
    return {name: onv.quantize_layer(m) for name, m in zip(("gate", "up", "down"), ms)}


def pin_bruteforce_layer(x, layer, ids, w, tol=1e-12):
    """Per-token pure-Python loops against the vectorised oracle."""
    out = omoe.moe_forward(x, layer, ids, w)
    t_all, h_dim = x.shape
    deq = {}
    for t in range(t_all):
        ref = [0.0] * h_dim
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if e not in deq:
                deq[e] = [a.astype(np.float64).tolist() for a in omoe.dequantize_expert(layer, e)]
            wg, wu, wd = deq[e]
            xt = [float(v) for v in x[t]]
            hvec = []
            for i in range(len(wg)):
                a = math.fsum(xt[q] * wg[i][q] for q in range(h_dim))
                b = math.fsum(xt[q] * wu[i][q] for q in range(h_dim))
                hvec.append(a / (1.0 + math.exp(-a)) * b)
            for n in range(h_dim):
                ref[n] += float(w[t, j]) * math.fsum(hvec[i] * wd[n][i] for i in range(len(hvec)))
        err = max(abs(a - b) for a, b in zip(out[t], ref))
        scale = max(abs(v) for v in ref)
        assert err <= tol * max(scale, 1e-300), (t, err, scale)


def pin_textbook_mlp(seed=0, H=64, I=32, T=5):
    """E = 1, k = 1: the layer is a plain SwiGLU MLP (torch fp64 on the CPU)."""
    r = np.random.default_rng(seed)
    ms = [(0.05 * r.standard_normal((1,) + s)).astype(np.float32)
          for s in ((I, H), (I, H), (H, I))]
    layer = _pack_layer(ms)
    x = r.standard_normal((T, H)).astype(np.float32)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1))
    out = omoe.moe_forward(x, layer, ids, w)
    wg, wu, wd = (torch.from_numpy(onv.dequantize(*[layer[p][i][0] for i in range(2)], layer[p][2][0])).double()
                  for p in ("gate", "up", "down"))
    xt = torch.from_numpy(x).double()
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xt, wg)) * torch.nn.functional.linear(xt, wu), wd)
    assert torch.allclose(torch.from_numpy(out), ref, rtol=1e-12, atol=1e-14)


def pin_one_hot_columns(seed=0, H=64, I=32):
    """A one-hot activation e_i reads column i of each weight: the gate and up
    pre-activations equal the weights at k = i, decoded here straight from
    the packed bytes (byte i // 2, nibble i % 2, scale i // 16)."""
    r = np.random.default_rng(seed)
    ms = [(0.05 * r.standard_normal((1,) + s)).astype(np.float32)
          for s in ((I, H), (I, H), (H, I))]
    layer = _pack_layer(ms)
    table = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    s_tab = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()

    def column(p, i):
        codes, scales, g = layer[p][0][0], layer[p][1][0], layer[p][2][0]
        byte = codes[:, i // 2]
        nib = (byte >> 4) if i % 2 else (byte & 15)
        # (c * s) is exact in fp32; the one rounding is at * g, in fp32
        cs = (table[nib] * s_tab[scales[:, i // 16]]).astype(np.float32)
        return (cs * np.float32(g)).astype(np.float64)

    wd = onv.dequantize(layer["down"][0][0], layer["down"][1][0], layer["down"][2][0]).astype(np.float64)
    for i in (0, 1, 2, 17, H - 1):
        x = np.zeros((1, H), np.float32)
        x[0, i] = 1.0
        out = omoe.moe_forward(x, layer, np.zeros((1, 1), np.int32), np.ones((1, 1)))
        a, b = column("gate", i), column("up", i)
        h = a / (1 + np.exp(-a)) * b
        assert np.allclose(out[0], wd @ h, rtol=1e-12, atol=1e-15)


def pin_magnitude(x, layer, ids, w, ms):
    """Nonzero output for every touched expert, and the quantized layer's
    output norm within [0.8, 1.25] of the unquantized fp64 layer's.  This is
    the guard against the zero-scale fault ("GLM-5.3-Flash on Blackwell",
    "The model loaded, served an API, and produced garbage"): an output scaled
    by zero, or by a wrong factor, fails here even when it correlates."""
    out = omoe.moe_forward(x, layer, ids, w)
    x64 = np.asarray(x, np.float64)
    for e in np.unique(ids):
        wg, wu, wd = omoe.dequantize_expert(layer, int(e))
        y = omoe.expert_ffn(x64[:1], wg, wu, wd)
        assert np.linalg.norm(y) > 0, e
    ref = np.zeros_like(x64)
    for t in range(x.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            ref[t] += w[t, j] * omoe.expert_ffn(x64[t:t + 1], ms[0][e], ms[1][e], ms[2][e])[0]
    ratio = float(np.linalg.norm(out) / np.linalg.norm(ref))
    assert 0.8 <= ratio <= 1.25, ratio
    rel = float(np.linalg.norm(out - ref) / np.linalg.norm(ref))
    assert rel < 0.25, rel
    return ratio, rel


def pin_linear_exact(seed=0):
    """The dense projection of an exactly representable weight equals x . W^T
    computed from that weight directly (no dequantization involved), and
    one-hot rows read out its columns (orientation and K indexing)."""
    w, _, _, _ = representable_tensor(seed)
    packed, scales, g = onv.quantize(w)
    r = np.random.default_rng(seed + 1)
    x = r.standard_normal((5, w.shape[1]))
    ref = x @ w.astype(np.float64).T
    got = omoe.linear(x, packed, scales, g)
    assert got.shape == (5, w.shape[0])
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    eye = np.eye(w.shape[1])
    assert np.array_equal(omoe.linear(eye, packed, scales, g), w.astype(np.float64).T)


def pin_shared_expert_textbook(seed=0, H=64, I=32, T=5):
    """The shared expert is a plain SwiGLU MLP (torch fp64 on the CPU) and the
    same as the routed layer with one expert, k = 1, weight 1."""
    r = np.random.default_rng(seed)
    ms = [(0.05 * r.standard_normal((1,) + s)).astype(np.float32)
          for s in ((I, H), (I, H), (H, I))]
    layer = _pack_layer(ms)
    x = r.standard_normal((T, H)).astype(np.float32)
    out = omoe.shared_expert_forward(x, layer)
    wg, wu, wd = (torch.from_numpy(onv.dequantize(*[layer[p][i][0] for i in range(2)], layer[p][2][0])).double()
                  for p in ("gate", "up", "down"))
    xt = torch.from_numpy(x).double()
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xt, wg)) * torch.nn.functional.linear(xt, wu), wd)
    assert torch.allclose(torch.from_numpy(out), ref, rtol=1e-12, atol=1e-14)
    routed = omoe.moe_forward(x, layer, np.zeros((T, 1), np.int32), np.ones((T, 1)))
    assert np.array_equal(out, routed)


# ---------------------------------------------------------------- W4A4 (activations in NVFP4 too)
from oracle import w4a4 as ow4  # noqa: E402


def _e4m3_bits_torch(x):
    """E4M3 bytes of non-negative fp32 values by torch's conversion, with the
    saturation at 448 applied first (torch maps >= 464 to NaN)."""
    x = np.minimum(np.asarray(x, np.float32), np.float32(448.0))
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_value_torch(b):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(b, np.uint8))).view(
        torch.float8_e4m3fn).to(torch.float32).numpy()


def _bruteforce_act_quant(row, input_scale):
    """One activation row -> its dequantized fp32 values, element by element:
    scale by torch's E4M3 conversion, code by a nearest search over the eight
    magnitudes (ties to the even code), sign copied from the quotient."""
    s_in = np.float32(input_scale)
    out = []
    for j in range(0, len(row), 16):
        grp = [np.float32(v) for v in row[j:j + 16]]
        amax = max(abs(v) for v in grp)
        s_f = np.float32(np.float32(amax / np.float32(6.0)) / s_in)
        s_q = _e4m3_value_torch(_e4m3_bits_torch([s_f]))[0]
        d = np.float32(s_q * s_in)
        for v in grp:
            if d == 0:
                out.append(0.0)
                continue
            q = np.float32(v / d)
            dist = [abs(abs(float(q)) - m) for m in E2M1_TABLE]
            best = [i for i, dd in enumerate(dist) if dd == min(dist)]
            c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            mag = E2M1_TABLE[c]
            val = np.float32(np.float32(mag * s_q) * s_in)
            out.append(-float(val) if np.signbit(q) else float(val))
    return out


def pin_act_exact_roundtrip(seed=0):
    """Activations built as code * E4M3 scale * input_scale (a +-6 code in
    every group, one group at scale 448) quantize back to exactly those codes
    and scales under that input scale, and dequantize to the same bits."""
    a, codes, sb, g = representable_tensor(seed)       # g = 2^-12 plays the input scale
    packed, scales = ow4.quantize_activations(a, g)
    assert np.array_equal(scales, sb)
    assert np.array_equal(onv.unpack_codes(packed), codes)
    back = ow4.dequantize_activations(packed, scales, g)
    assert np.array_equal(back.view(np.uint32), a.view(np.uint32))
    # the same tensor under twice the input scale: every scale byte halves
    # its value (one binade down), codes unchanged -- the scale is used, once
    p2, s2 = ow4.quantize_activations(a, np.float32(2 * g))
    normal = np.repeat(sb >= 0x10, 16, axis=1)        # groups whose halved scale stays normal
    assert np.array_equal(onv.unpack_codes(p2)[normal], codes[normal])
    assert np.array_equal(_e4m3_value_torch(s2[sb >= 0x10]) * 2, _e4m3_value_torch(sb[sb >= 0x10]))


def pin_act_scale_rule(seed=0, input_scale=np.float32(6.0 / 2688.0)):
    """Group scales of random activations against torch's E4M3 conversion of
    (amax / 6) / input_scale, and every dequantized value against the
    element-by-element brute force."""
    r = np.random.default_rng(seed)
    a = r.standard_normal((6, 96)).astype(np.float32)
    a[1, :16] = 0.0
    a[2, 16:32] = np.float32(1e-4) * a[2, 16:32]             # small-amax group
    a[3, 40] = np.float32(50.0)                                # beyond 6 * 448 * s: saturates
    packed, scales = ow4.quantize_activations(a, input_scale)
    amax_g = np.abs(a).reshape(6, 6, 16).max(axis=2)
    s_f = (amax_g / np.float32(6)) / np.float32(input_scale)
    assert np.array_equal(scales, _e4m3_bits_torch(s_f))
    got = ow4.dequantize_activations(packed, scales, input_scale)
    for i in range(a.shape[0]):
        assert got[i].tolist() == _bruteforce_act_quant(a[i], input_scale), i


def pin_input_scale_refusal():
    """Missing, zero, negative and non-finite input scales are refused, by the
    quantizer and by the layer (the unset-scale fault)."""
    x = np.ones((2, 32), np.float32)
    layer = _pack_layer([np.full((1, 32, 32), 0.01, np.float32)] * 3)
    ids, w = np.zeros((2, 1), np.int32), np.ones((2, 1))
    for bad in (None, 0.0, -0.0, -1.0, float("nan"), float("inf"), float("-inf")):
        for call in (lambda: ow4.quantize_activations(x, bad),
                     lambda: ow4.moe_forward_w4a4(x, layer, ids, w, bad, 1.0),
                     lambda: ow4.moe_forward_w4a4(x, layer, ids, w, 1.0, bad)):
            try:
                call()
            except ValueError:
                continue
            raise AssertionError(f"input scale {bad!r} accepted")


def pin_placeholder_underflow():
    """The placeholder input scale 1.0 the pages report: a group whose
    amax / 6 falls below half the smallest E4M3 step (2^-10) gets scale 0 and
    all-zero activations, so a token of small activations yields an exactly
    zero layer output; a calibrated scale (amax / 2688) keeps it, close to
    the W4A16 output."""
    r = np.random.default_rng(3)
    H, I = 64, 32
    ms = [(0.05 * r.standard_normal((1,) + s)).astype(np.float32) for s in ((I, H), (I, H), (H, I))]
    layer = _pack_layer(ms)
    x = (np.float32(5e-4) * r.standard_normal((1, H))).astype(np.float32)   # amax / 6 < 2^-10
    ids, w = np.zeros((1, 1), np.int32), np.ones((1, 1))
    packed, scales = ow4.quantize_activations(x, 1.0)
    assert not scales.any() and not (onv.unpack_codes(packed) & 7).any()
    assert not ow4.moe_forward_w4a4(x, layer, ids, w, 1.0, 1.0).any()
    cal = np.float32(np.max(np.abs(x)) / np.float32(2688.0))
    y = ow4.moe_forward_w4a4(x, layer, ids, w, cal, 1.0e-6)
    ref = omoe.moe_forward(x, layer, ids, w)
    assert np.linalg.norm(y) > 0
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.35


def pin_w4a4_representable_x(seed=0):
    """Activations exactly representable under their input scale pass the
    quantizer unchanged, so the W4A4 gate/up pre-activations and h equal the
    W4A16 layer's on the same x."""
    r = np.random.default_rng(seed)
    H, I = 96, 32
    xa, _, _, g = representable_tensor(seed, n=3, k=H)
    ms = [(0.05 * r.standard_normal((1,) + s)).astype(np.float32) for s in ((I, H), (I, H), (H, I))]
    layer = _pack_layer(ms)
    wg, wu, wd = omoe.dequantize_expert(layer, 0)
    xq = ow4.fake_quantize(xa, g)
    assert np.array_equal(xq.view(np.uint32), xa.view(np.uint32))
    _, h = ow4.expert_ffn_w4a4(xq, wg, wu, wd, np.float32(1.0), return_h=True)
    x64 = xa.astype(np.float64)
    a, b = x64 @ wg.astype(np.float64).T, x64 @ wu.astype(np.float64).T
    assert np.array_equal(h, a / (1.0 + np.exp(-a)) * b)


def pin_w4a4_bruteforce(seed=0, H=64, I=64, E=4, k=2, T=16, tol=1e-12):
    """Per-token pure-Python loops (their own activation quantizer, math.fsum
    products) against the vectorised W4A4 oracle on a tiny layer."""
    r = np.random.default_rng(seed)
    ms = [(0.05 * r.standard_normal((E,) + s)).astype(np.float32) for s in ((I, H), (I, H), (H, I))]
    layer = _pack_layer(ms)
    x = r.standard_normal((T, H)).astype(np.float32)
    lg = r.standard_normal((T, E)).astype(np.float32)
    ids, w = ort.route_topk(lg, k)
    sx, sh = np.float32(5.0 / 2688.0), np.float32(3.0 / 2688.0)
    out = ow4.moe_forward_w4a4(x, layer, ids, w, sx, sh)
    deq = {}
    for t in range(T):
        xq = _bruteforce_act_quant(x[t], sx)
        ref = [0.0] * H
        for j in range(k):
            e = int(ids[t, j])
            if e not in deq:
                deq[e] = [a.astype(np.float64).tolist() for a in omoe.dequantize_expert(layer, e)]
            wg, wu, wd = deq[e]
            hvec = []
            for i in range(I):
                a = math.fsum(xq[q] * wg[i][q] for q in range(H))
                b = math.fsum(xq[q] * wu[i][q] for q in range(H))
                hvec.append(np.float32(a / (1.0 + math.exp(-a)) * b))
            hq = _bruteforce_act_quant(hvec, sh)
            for n in range(H):
                ref[n] += float(w[t, j]) * math.fsum(hq[i] * wd[n][i] for i in range(I))
        err = max(abs(a - b) for a, b in zip(out[t], ref))
        assert err <= tol * max(max(abs(v) for v in ref), 1e-300), (t, err)


def pin_w4a4_magnitude(seed=0, H=128, I=64, E=4, k=2, T=16):
    """The W4A4 output keeps the unquantized layer's magnitude (norm ratio in
    [0.8, 1.25]) and differs from the W4A16 output by the activation
    quantization error -- clearly nonzero, well below the signal."""
    r = np.random.default_rng(seed)
    ms = [(0.02 * r.standard_normal((E,) + s)).astype(np.float32) for s in ((I, H), (I, H), (H, I))]
    layer = _pack_layer(ms)
    x = r.standard_normal((T, H)).astype(np.float32)
    ids, w = ort.route_topk(r.standard_normal((T, E)).astype(np.float32), k)
    sx = np.float32(np.max(np.abs(x)) / np.float32(2688.0))
    h_amax = 0.0
    for e in range(E):
        wg, wu, _ = omoe.dequantize_expert(layer, e)
        a, b = x.astype(np.float64) @ wg.T.astype(np.float64), x.astype(np.float64) @ wu.T.astype(np.float64)
        h_amax = max(h_amax, float(np.max(np.abs(a / (1 + np.exp(-a)) * b))))
    sh = np.float32(np.float32(h_amax) / np.float32(2688.0))
    y4 = ow4.moe_forward_w4a4(x, layer, ids, w, sx, sh)
    y16 = omoe.moe_forward(x, layer, ids, w)
    x64 = x.astype(np.float64)
    ref = np.zeros_like(x64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            ref[t] += w[t, j] * omoe.expert_ffn(x64[t:t + 1], ms[0][e], ms[1][e], ms[2][e])[0]
    ratio = float(np.linalg.norm(y4) / np.linalg.norm(ref))
    assert 0.8 <= ratio <= 1.25, ratio
    d = float(np.linalg.norm(y4 - y16) / np.linalg.norm(y16))
    assert 0.01 <= d <= 0.3, d
    return ratio, d
