"""Router top-k with softmax weights, and the expert-sorted permutation.
TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say only that every MoE layer has a BF16 router that is never
quantized ("GLM-5.3-Flash on Blackwell", "The quantization";
"GLM-5.3-Flash-NVFP4-h", "Config expectations" lists the 42 per-layer
``mlp.gate`` routers as excluded).  Readings used here:

* the router logits arrive as fp32 [T, E] (the router GEMM is not on this
  path);
* per token, experts are ordered by (logit descending, expert index
  ascending) and the first k are selected, in that order;
* the routing weights are a softmax over the k selected logits, in fp64,
  which equals a softmax over all E followed by renormalisation over the
  selected k;
* no bias correction, no grouped top-k, no routed scaling factor.

Permutation: ``counts[e]`` is the number of (token, slot) pairs routed to e;
``offsets`` its exclusive prefix sum with ``offsets[E] = T*k``;
``sorted_slots`` lists the flat indices ``t*k + j`` grouped by expert, in
ascending flat index inside each expert (a stable counting sort);
``slot_pos`` is its inverse.

Pins (tests/test_oracle_routing.py): a brute-force per-token sort with
Python's ``sorted``, weights summing to 1, the softmax-all-then-renormalise
identity, and the permutation checked against Python ``sorted`` on
(expert, flat index) plus bijection and count invariants.
"""

import numpy as np


def route_topk(logits, k):
    """Return ``(ids int32 [T, k], weights float64 [T, k])``."""
    logits = np.asarray(logits, dtype=np.float32)
    t, e = logits.shape
    if not 1 <= k <= e:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((t, k), dtype=np.int32)
    weights = np.empty((t, k), dtype=np.float64)
    index = np.arange(e)
    for row in range(t):
        order = np.lexsort((index, -logits[row].astype(np.float64)))
        sel = order[:k]
        ids[row] = sel
        sel_logits = logits[row, sel].astype(np.float64)
        ex = np.exp(sel_logits - sel_logits.max())
        weights[row] = ex / ex.sum()
    return ids, weights


def permutation(ids, num_experts):
    """Stable expert-major permutation of the flat (token, slot) indices.

    Returns ``(counts [E], offsets [E+1], sorted_slots [T*k], slot_pos [T*k])``,
    all int32.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=num_experts)[:num_experts]
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_slots = np.argsort(flat, kind="stable")
    slot_pos = np.empty_like(sorted_slots)
    slot_pos[sorted_slots] = np.arange(flat.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_slots.astype(np.int32), slot_pos.astype(np.int32))
