"""Seeded synthetic inputs for the five MoE-layer workloads.

This module holds no arithmetic of the method: it only draws random numbers
and rounds the activations to their storage type.  Both the HIP library's
tests/bench and the CPU oracle consume what it produces; neither side's
arithmetic lives here.

Recipe (numpy ``Generator(PCG64(SeedSequence(key)))``, seed 0 first in every
key):

* master weights: ``0.02 * standard_normal(float32)`` per (projection,
  expert), shape [N, K] row-major, key ``[0, wset, proj, e]`` with proj
  0/1/2 = gate/up/down.  ``wset`` 0 is the tiny layer; ``wset`` 1 is the one
  full-size layer shared by the four full-size workloads;
* activations: fp32 ``standard_normal`` [T, H], key ``[0, cfg, 3]``, rounded
  to bf16 (round to nearest even);
* router logits: fp32 ``standard_normal`` [T, E], key ``[0, cfg, 4]``, plus a
  per-workload bias:
  - ``shared``: one bias vector shared by every token, +2.0 on 8 experts drawn
    without replacement (key ``[0, cfg, 5]``), so the tokens of a decode batch
    overlap on some experts;
  - ``zipf``: ``b_e = -1.1 * ln(r_e)`` with ``r = permutation(E) + 1`` (key
    ``[0, cfg, 5]``), which makes the expert prior proportional to
    ``r_e ** -1.1`` (Zipf, s = 1.1): a few hot experts with thousands of
    tokens and many cold ones near zero.

The shapes are those of a GLM-5.3-Flash-class routed-expert layer: hidden
5120, 256 experts, top-8, intermediate 1536.

W4A4 input scales: a W4A4 checkpoint carries static, calibrated activation
scales; the synthetic stand-ins are fixed constants, one for the gate/up
input (covering |x| <= 6 of the N(0, 1) activations at the largest code and
scale) and one for the down input (covering |h| <= 32).
"""

from dataclasses import dataclass

import numpy as np

GATE, UP, DOWN = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    wset: int
    bias: str  # "none" | "shared" | "zipf"


WORKLOADS = {
    0: Workload(0, "tiny-moe-t16-h256-i128-e8-k2", 16, 256, 128, 8, 2, 0, "none"),
    1: Workload(1, "decode-t1-h5120-i1536-e256-k8", 1, 5120, 1536, 256, 8, 1, "none"),
    2: Workload(2, "decode-mtp-t8-h5120-i1536-e256-k8-sharedbias", 8, 5120, 1536, 256, 8, 1, "shared"),
    3: Workload(3, "prefill-t1024-h5120-i1536-e256-k8", 1024, 5120, 1536, 256, 8, 1, "none"),
    4: Workload(4, "prefill-t16384-h5120-i1536-e256-k8-zipf1.1", 16384, 5120, 1536, 256, 8, 1, "zipf"),
}


# (gate/up input, down input) static input scales of the W4A4 workloads
W4A4_INPUT_SCALES = (2.2321428e-03, 1.1904762e-02)


def rng(key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def proj_shape(wl, proj):
    """(N, K) of a projection: gate/up map H -> I, down maps I -> H."""
    return (wl.I, wl.H) if proj in (GATE, UP) else (wl.H, wl.I)


def master(wl, proj, e, scale=0.02):
    """fp32 master weights [N, K] of one (projection, expert)."""
    n, k = proj_shape(wl, proj)
    w = rng((0, wl.wset, proj, e)).standard_normal(size=(n, k), dtype=np.float32)
    w *= np.float32(scale)
    return w


def masters(wl, proj, experts=None):
    """Stack of masters [len(experts), N, K] (all experts by default)."""
    experts = range(wl.E) if experts is None else experts
    return np.stack([master(wl, proj, e) for e in experts])


def activations_fp32(wl, T=None):
    T = wl.T if T is None else T
    return rng((0, wl.cfg, 3)).standard_normal(size=(T, wl.H), dtype=np.float32)


def to_bf16_bits(a):
    """Round fp32 values to bf16 (nearest even) and return the uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact fp32 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def activations(wl, T=None):
    """(bf16 bits uint16 [T, H], the same values as fp32)."""
    bits = to_bf16_bits(activations_fp32(wl, T))
    return bits, bf16_bits_to_f32(bits)


def router_bias(wl):
    if wl.bias == "none":
        return np.zeros(wl.E, dtype=np.float32)
    g = rng((0, wl.cfg, 5))
    if wl.bias == "shared":
        b = np.zeros(wl.E, dtype=np.float32)
        b[g.choice(wl.E, 8, replace=False)] = np.float32(2.0)
        return b
    if wl.bias == "zipf":
        r = g.permutation(wl.E) + 1
        return (-1.1 * np.log(r.astype(np.float64))).astype(np.float32)
    raise ValueError(wl.bias)


def logits(wl, T=None):
    """fp32 router logits [T, E] including the workload's bias."""
    T = wl.T if T is None else T
    z = rng((0, wl.cfg, 4)).standard_normal(size=(T, wl.E), dtype=np.float32)
    return (z + router_bias(wl)[None, :]).astype(np.float32)


def random_problem(seed, T, H, I, E, k):
    """Small random problem for shape sweeps: (wl, masters per proj, x bits,
    x fp32, logits).  Keys start with 1 so they never collide with the
    workloads above."""
    wl = Workload(-1, f"random-{seed}", T, H, I, E, k, 1000 + seed, "none")
    g = rng((1, seed))
    ms = []
    for proj in (GATE, UP, DOWN):
        n, kk = proj_shape(wl, proj)
        ms.append((np.float32(0.02) * g.standard_normal(size=(E, n, kk), dtype=np.float32)))
    xb = to_bf16_bits(g.standard_normal(size=(T, H), dtype=np.float32))
    lg = g.standard_normal(size=(T, E), dtype=np.float32)
    return wl, ms, xb, bf16_bits_to_f32(xb), lg


def router_problem(seed, T, H, E):
    """BF16 router inputs: (x bits [T, H], x fp32, router weight bits [E, H],
    router weight fp32).  x ~ N(0, 1) and weights ~ N(0, 1/H) rounded to bf16,
    so the logits are about N(0, 1) like the drawn logits of the workloads.
    Keys start with 2 so they never collide with the generators above."""
    g = rng((2, seed))
    xb = to_bf16_bits(g.standard_normal(size=(T, H), dtype=np.float32))
    wb = to_bf16_bits(np.float32(1.0 / np.sqrt(H)) * g.standard_normal(size=(E, H), dtype=np.float32))
    return xb, bf16_bits_to_f32(xb), wb, bf16_bits_to_f32(wb)
