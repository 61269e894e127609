"""CPU oracle for the NVFP4 weight-only (W4A16) routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test-suite, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or helper with the HIP library in ``nvfp4_weight_only_moe_amd``; the two meet
only through the seeded input generators of ``nvfp4_weight_only_moe_amd.workloads``.

The oracle is plain and slow on purpose: numpy, fp64 for the FFN, and the
exact fp32 operations where the format itself fixes fp32 (the scales and the
integer codes they decide).

Sources (page title and section; no page prints formulas or code):

* "GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side quantization", intro and
  "Config expectations": weight-only 4-bit NVFP4 with group size 16, and an
  FP32 per-tensor second-level scale (``weight_scale_2``) that must be present.
* "GLM-5.3-Flash on Blackwell", "The quantization": routed experts are stored
  as separate per-expert, per-projection 4-bit tensors; routers stay BF16.
* same page, "The model loaded, served an API, and produced garbage": a
  weight-only checkpoint ships no activation scale, the W4A16 route dequantises
  weights to bf16, and a kernel is checked against an fp32 reference on
  magnitude, not on correlation alone.
* "GLM-5.3-Flash NVFP4 W4A16 for 2x RTX PRO 6000 Blackwell", intro: the routed
  experts are W4A16_NVFP4 and need no activation calibration.

The pages never print the E2M1/E4M3 bit layouts, the scale formulas, the
router function or the activation.  Those are fixed here as readings:
E2M1 and E4M3 ("FN", no infinities) follow the OCP Microscaling v1.0 and OCP
8-bit floating point specifications; the two-level scale is
``g = amax(tensor) / (6 * 448)`` and ``s = E4M3((amax(group) / 6) / g)``;
routing is softmax over the top-k logits; the expert FFN is SwiGLU.

Parity status per function is stated in each module's docstring.
"""

from .formats import (E2M1_MAGNITUDES, e2m1_decode, e2m1_encode, e4m3_decode,
                      e4m3_encode)
from .nvfp4 import quantize, dequantize, quantize_layer
from .routing import route_topk, permutation
from .moe import moe_forward, expert_ffn
from .router import router_logits

__all__ = [
    "E2M1_MAGNITUDES", "e2m1_decode", "e2m1_encode", "e4m3_decode",
    "e4m3_encode", "quantize", "dequantize", "quantize_layer", "route_topk",
    "permutation", "moe_forward", "expert_ffn", "router_logits",
]
