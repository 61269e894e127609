"""NVFP4 weight-only quantization and dequantization of one [N, K] tensor.
TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: 4-bit weight-only NVFP4, group size 16 along the input
(K) dimension, and one FP32 second-level scale per quantized tensor
("GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side quantization", "Config
expectations"); routed experts are separate per-expert, per-projection
tensors ("GLM-5.3-Flash on Blackwell", "The quantization"); the conversion is
deterministic and needs no calibration data ("GLM-5.3-Flash NVFP4 W4A16 for
2x RTX PRO 6000 Blackwell", intro).

Readings (the pages print no formula), all in fp32 with one correctly rounded
operation per step, in this order:

1. ``amax_t = max |W|`` over the tensor (exact).
2. ``g = amax_t / 2688`` (2688 = 6 * 448, the largest E2M1 magnitude times
   the largest E4M3 value).  If that is 0 -- an all-zero tensor, or one so
   small that the quotient underflows -- ``g = 1``, so the stored global scale
   is always a positive finite number and an unset (zero) scale stays
   detectable.
3. Per group of 16 consecutive k in a row: ``amax_g = max |W|``,
   ``s_f = (amax_g / 6) / g``, ``s_b = E4M3(s_f)`` (nearest, ties to even,
   saturating), ``s_q`` its value.
4. ``d = s_q * g``.  If ``d == 0`` every code of the group has magnitude 0 and
   keeps the sign bit of its weight.  Otherwise ``c = E2M1(W / d)``.
5. Packing: byte ``i`` of a row holds code ``2i`` in its low nibble and code
   ``2i + 1`` in its high nibble; the scale bytes form their own row-major
   ``[N, K/16]`` array.

Dequantization: ``W' = (E2M1(c) * E4M3(s)) * g`` in fp32.  The first product
is exact (at most 6 significant bits); the only rounding is the one at ``* g``.

Pins: exact round-trip of representable tensors, one-hot and sign/zero cases,
all-zero and underflowing tensors, nibble order, and the soft round-trip
cosine band (tests/test_oracle_quant.py).
"""

import numpy as np

from .formats import e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode

GROUP = 16
GLOBAL_DIVISOR = np.float32(6.0 * 448.0)


def global_scale(amax_t):
    """Step 2: fp32 global scale from the tensor's fp32 absolute maximum."""
    g = np.float32(amax_t) / GLOBAL_DIVISOR
    if not g > 0:
        g = np.float32(1.0)
    return np.float32(g)


def quantize(w):
    """Quantize one fp32 tensor ``w`` of shape [N, K] (K % 32 == 0).

    Returns ``(codes, scales, g)``: codes uint8 [N, K/2] (two nibbles per
    byte), scales uint8 [N, K/16] (E4M3 bit patterns), g a float32 scalar.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % 32:
        raise ValueError("quantize expects [N, K] with K % 32 == 0")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite master weight")
    n, k = w.shape
    g = global_scale(np.max(np.abs(w)) if w.size else np.float32(0))
    packed = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty((n, k // GROUP), dtype=np.uint8)
    rows = max(1, (1 << 16) // k)          # a few rows at a time keeps temporaries small
    for r0 in range(0, n, rows):
        packed[r0:r0 + rows], scales[r0:r0 + rows] = _quantize_rows(w[r0:r0 + rows], g)
    return packed, scales, np.float32(g)


def _quantize_rows(w, g):
    """Steps 3-5 for a block of rows with the tensor's global scale ``g``."""
    n, k = w.shape
    groups = w.reshape(n, k // GROUP, GROUP)
    amax_g = np.max(np.abs(groups), axis=2)
    s_f = (amax_g / np.float32(6.0)) / g                       # two fp32 divides
    s_b = e4m3_encode(s_f)
    s_q = e4m3_decode(s_b).astype(np.float32)
    d = (s_q * g).astype(np.float32)

    with np.errstate(divide="ignore", invalid="ignore"):
        q = groups / d[:, :, None]                             # fp32 divide
    zero_group = (d == 0)[:, :, None]
    q = np.where(zero_group, np.where(np.signbit(groups), np.float32(-0.0),
                                      np.float32(0.0)), q).astype(np.float32)
    codes = e2m1_encode(q).reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_b.astype(np.uint8)


def unpack_codes(packed):
    """[N, K/2] packed bytes -> [N, K] codes, even k from the low nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, half = packed.shape
    codes = np.empty((n, half * 2), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes


def dequantize(packed, scales, g):
    """fp32 [N, K] weights from one packed tensor: (E2M1 * E4M3) * g."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, k = packed.shape[0], packed.shape[1] * 2
    out = np.empty((n, k), dtype=np.float32)
    rows = max(1, (1 << 16) // k)          # a few rows at a time keeps temporaries small
    for r0 in range(0, n, rows):
        codes = unpack_codes(packed[r0:r0 + rows])
        m = codes.shape[0]
        c = e2m1_decode(codes).astype(np.float32).reshape(m, k // GROUP, GROUP)
        s = e4m3_decode(scales[r0:r0 + rows]).astype(np.float32)[:, :, None]
        w = (c * s).astype(np.float32) * np.float32(g)
        out[r0:r0 + rows] = w.reshape(m, k)
    return out


def quantize_layer(masters):
    """Quantize a stack of per-expert tensors [E, N, K]; returns
    ``(codes [E, N, K/2], scales [E, N, K/16], g [E])``."""
    packed, scales, gs = [], [], []
    for w in masters:
        p, s, g = quantize(w)
        packed.append(p)
        scales.append(s)
        gs.append(g)
    return np.stack(packed), np.stack(scales), np.asarray(gs, dtype=np.float32)
