"""The routed-expert MoE layer with dequantized NVFP4 weights, in fp64.
TEST INFRASTRUCTURE ONLY (see the package docstring).

Plain definition (a reading: the pages name gate/up/down projections --
"GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side quantization", intro -- but not
the activation, which is taken to be SwiGLU):

    out[t] = sum_j  w[t, j] * FFN_{e(t, j)}(x[t])
    FFN_e(x) = (silu(x @ Wg_e^T) * (x @ Wu_e^T)) @ Wd_e^T,  silu(a) = a / (1 + exp(-a))

with ``Wg_e, Wu_e, Wd_e`` the dequantized fp32 weights of expert e
(``oracle.nvfp4.dequantize``) taken exactly into fp64, ``x`` the bf16
activations taken exactly into fp64, and every product and sum in fp64.
The W4A16 route needs no activation scale and the layer takes none
("GLM-5.3-Flash on Blackwell", "The model loaded, served an API, and produced
garbage").

Experts are visited one at a time in ascending index and each adds
``w * y`` into an fp64 output, so memory stays bounded at any size; within a
token the k terms are added in that expert order (exact up to fp64 rounding).

``round_h_bf16=True`` is a diagnostic: it rounds the SwiGLU output to bf16
(fp64 -> fp32 -> bf16, RNE) before the down projection, mimicking the
device's one bf16 intermediate so that small device bugs stand out.

Pins (tests/test_oracle_moe.py): brute-force per-token loops on the tiny
configuration, reduction to a textbook SwiGLU MLP (torch fp64) for E = 1,
k = 1, one-hot activations that read out single weight columns (nibble order
and K indexing), and the magnitude checks (nonzero expert output; norm ratio
to the unquantized layer).
"""

import numpy as np
import torch

from .nvfp4 import dequantize


def silu(a):
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def _bf16_round(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def expert_ffn(x, wg, wu, wd, round_h_bf16=False):
    """SwiGLU FFN of one expert in fp64: rows of ``x`` [M, H] -> [M, H]."""
    x = np.asarray(x, dtype=np.float64)
    a = x @ np.asarray(wg, dtype=np.float64).T
    b = x @ np.asarray(wu, dtype=np.float64).T
    h = silu(a) * b
    if round_h_bf16:
        h = _bf16_round(h)
    return h @ np.asarray(wd, dtype=np.float64).T


def dequantize_expert(layer, e):
    """fp32 (Wg, Wu, Wd) of expert ``e`` from a packed layer dict
    ``{"gate": (codes, scales, g), "up": ..., "down": ...}``."""
    return tuple(dequantize(layer[p][0][e], layer[p][1][e], layer[p][2][e])
                 for p in ("gate", "up", "down"))


def moe_forward(x, layer, ids, weights, tokens=None, round_h_bf16=False):
    """fp64 [T, H] layer output (rows not in ``tokens`` are left at zero).

    x: [T, H] activations (the bf16 values, any float dtype that holds them
    exactly); layer: packed layer dict; ids [T, k] expert ids; weights [T, k]
    routing weights; tokens: optional iterable of token indices to compute.
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    weights = np.asarray(weights, dtype=np.float64)
    t_all, _ = x.shape
    tokens = np.arange(t_all) if tokens is None else np.asarray(sorted(set(int(t) for t in tokens)))
    out = np.zeros_like(x)
    experts = np.unique(ids[tokens].reshape(-1)) if tokens.size else []
    for e in experts:
        rows, slots = np.nonzero(ids[tokens] == e)
        toks = tokens[rows]
        wg, wu, wd = dequantize_expert(layer, int(e))
        y = expert_ffn(x[toks], wg, wu, wd, round_h_bf16=round_h_bf16)
        out[toks] += weights[toks, slots][:, None] * y
    return out


def linear(x, codes, scales, g):
    """Dense projection in fp64: rows of ``x`` [M, K] times the transposed
    dequantized [N, K] weight -> [M, N].  The dense layers (attention
    linears, shared experts, lm_head) quantized to W4A16 NVFP4 like the
    experts: "GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side quantization", its
    opening.  Pinned against an exactly representable weight and one-hot rows
    (tests/test_oracle_moe.py)."""
    w = np.asarray(dequantize(codes, scales, g), dtype=np.float64)
    return np.asarray(x, dtype=np.float64) @ w.T


def shared_expert_forward(x, layer, round_h_bf16=False):
    """The shared expert: the SwiGLU FFN of expert 0 of ``layer`` for every
    row, with weight 1 (the model's single shared expert runs for every token
    beside the routed ones: "GLM-5.3-Flash on Blackwell", "The model loaded,
    served an API, and produced garbage").  Equal to ``moe_forward`` with
    E = 1, k = 1; pinned against a textbook SwiGLU MLP."""
    wg, wu, wd = dequantize_expert(layer, 0)
    return expert_ffn(x, wg, wu, wd, round_h_bf16=round_h_bf16)
