"""The W4A4 NVFP4 variant of the routed-expert layer: weights AND activations
in NVFP4.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:

* the stock routed experts of the NVIDIA release keep W4A4 NVFP4 -- 4-bit
  weights and 4-bit activations -- while a derivative moves the dense side to
  weight-only W4A16 ("GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side
  quantization", its opening paragraph);
* a W4A4 checkpoint ships a per-tensor activation scale (``input_scale``)
  for its experts; a placeholder of 1.0 made blocks of small activations
  underflow to zero and was replaced by a recalibrated one
  ("GLM-5.3-Flash · 512k + MTP + vision ...", "Input-scales provenance");
* an activation scale that is missing and read as an uninitialised 0.0
  multiplies every expert output by zero, so a missing or zero input scale
  must be refused loudly rather than computed with ("GLM-5.3-Flash on
  Blackwell", "The model loaded, served an API, and produced garbage").

Readings (the pages print no formula):

1. An activation row is quantized exactly like a weight row (oracle.nvfp4):
   groups of 16 consecutive k, one E4M3 scale per group, E2M1 codes, with the
   per-tensor FP32 ``input_scale`` in the place of the weight's global scale
   and the same fp32 operation order:
   ``s = E4M3((amax(group) / 6) / input_scale)``,
   ``code = E2M1(x / (E4M3(s) * input_scale))``.
   Dequantized: ``(E2M1(code) * E4M3(s)) * input_scale`` in fp32.
2. The input scale is a static, calibrated constant -- not derived from the
   batch -- with one FP32 value for the gate/up input ``x`` (gate and up read
   the same activations) and one for the down input ``h``.  It must be a
   finite number > 0; anything else (missing, 0, negative, NaN, inf) is
   refused with ValueError.
3. ``h = silu(a) * b`` is computed in fp64 as in the W4A16 layer, rounded
   once to fp32, and that fp32 value is quantized (no bf16 copy in between).
4. Everything else (routing, combine, fp64 products and sums) is the W4A16
   layer of oracle.moe.

Pins (tests/test_oracle_w4a4.py): exact round trip of activations built from
known codes and scales under a given input scale, the scale rule against
torch's E4M3 conversion and a brute-force nearest-code search, refusal of
every bad input scale, the placeholder-scale underflow the pages describe,
equality with the W4A16 layer's pre-activations for exactly representable
activations, pure-Python per-token loops on a tiny layer, and the magnitude
bands; planted mistakes in tests/test_oracle_mutations.py.
"""

import math

import numpy as np

from .moe import dequantize_expert, silu
from .nvfp4 import GROUP, _quantize_rows, dequantize


def check_input_scale(s, name="input_scale"):
    """The input scale as fp32, or ValueError when it is missing, not finite
    or not > 0 (the unset-scale fault)."""
    if s is None:
        raise ValueError(f"{name} is missing")
    v = np.float32(s)
    if not math.isfinite(float(v)):
        raise ValueError(f"{name} is not finite: {s!r}")
    if not float(v) > 0.0:
        raise ValueError(f"{name} must be > 0, got {s!r}")
    return v


def quantize_activations(a, input_scale):
    """fp32 activations [M, K] (K % 16 == 0) -> (codes uint8 [M, K/2] packed
    like the weights, scales uint8 [M, K/16] E4M3 bytes)."""
    s = check_input_scale(input_scale)
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim != 2 or a.shape[1] % 32:
        raise ValueError("quantize_activations expects [M, K] with K % 32 == 0")
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite activation")
    m, k = a.shape
    packed = np.empty((m, k // 2), dtype=np.uint8)
    scales = np.empty((m, k // GROUP), dtype=np.uint8)
    rows = max(1, (1 << 16) // k)
    for r0 in range(0, m, rows):
        packed[r0:r0 + rows], scales[r0:r0 + rows] = _quantize_rows(a[r0:r0 + rows], s)
    return packed, scales


def dequantize_activations(packed, scales, input_scale):
    """fp32 [M, K]: (E2M1 * E4M3) * input_scale, one rounding at the last
    product (the weight rule)."""
    return dequantize(packed, scales, check_input_scale(input_scale))


def fake_quantize(a, input_scale):
    """What the layer computes with: the activations quantized to NVFP4 and
    dequantized back, fp32 [M, K]."""
    return dequantize_activations(*quantize_activations(a, input_scale), input_scale)


def expert_ffn_w4a4(xq, wg, wu, wd, input_scale_h, return_h=False):
    """SwiGLU FFN of one expert on already quantized activations ``xq``
    (fp32 values of NVFP4 activations), with the hidden activations quantized
    to NVFP4 under ``input_scale_h`` before the down projection."""
    x = np.asarray(xq, dtype=np.float64)
    a = x @ np.asarray(wg, dtype=np.float64).T
    b = x @ np.asarray(wu, dtype=np.float64).T
    h = silu(a) * b
    hq = fake_quantize(h.astype(np.float32), input_scale_h).astype(np.float64)
    y = hq @ np.asarray(wd, dtype=np.float64).T
    return (y, h) if return_h else y


def moe_forward_w4a4(x, layer, ids, weights, input_scale_x, input_scale_h, tokens=None):
    """fp64 [T, H] output of the W4A4 layer (rows not in ``tokens`` stay 0).

    x: [T, H] activations (the bf16 values, exactly in fp32); layer: packed
    weight dict as for oracle.moe_forward; ids/weights: routing [T, k];
    input_scale_x / input_scale_h: the static FP32 input scales of the
    gate/up input and of the down input.
    """
    sx = check_input_scale(input_scale_x, "input_scale_x")
    sh = check_input_scale(input_scale_h, "input_scale_h")
    x = np.asarray(x, dtype=np.float32)
    ids = np.asarray(ids)
    weights = np.asarray(weights, dtype=np.float64)
    t_all = x.shape[0]
    tokens = np.arange(t_all) if tokens is None else np.asarray(sorted(set(int(t) for t in tokens)))
    out = np.zeros(x.shape, dtype=np.float64)
    if tokens.size == 0:
        return out
    xq = np.zeros(x.shape, dtype=np.float32)
    xq[tokens] = fake_quantize(x[tokens], sx)         # each token row is quantized once
    for e in np.unique(ids[tokens].reshape(-1)):
        rows, slots = np.nonzero(ids[tokens] == e)
        toks = tokens[rows]
        wg, wu, wd = dequantize_expert(layer, int(e))
        y = expert_ffn_w4a4(xq[toks], wg, wu, wd, sh)
        out[toks] += weights[toks, slots][:, None] * y
    return out
