"""Router logits: the BF16 gate of a MoE layer, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The routers are kept in BF16 and never quantized ("GLM-5.3-Flash on
Blackwell", "The quantization"; the per-layer ``mlp.gate`` modules are in the
ignore list of "GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side quantization",
"Config expectations"; and in the list of tensors the
GLM-5.3-Flash-NVFP4-FP8ATTN-512K model card keeps in BF16, "What exactly is
quantized").  The pages print no router
formula; the reading taken is the plain linear gate without bias,
``logits[t, e] = sum_i x[t, i] * W[e, i]`` over the hidden size, with bf16
inputs and the sum in fp64 here (the device sums in fp32).

Pinned in tests/test_oracle_router.py: one-hot rows pick single weights
exactly (indexing and orientation), constant rows against a closed form,
and the sign and scale under negation of the weights.
"""
import numpy as np


def router_logits(x, w_r):
    """fp64 logits [T, E] of rows ``x`` [T, H] under router weights ``w_r``
    [E, H] (both holding bf16 values)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_r, dtype=np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"router_logits: x {x.shape} and w_r {w.shape} must be [T, H] and [E, H]")
    return x @ w.T
