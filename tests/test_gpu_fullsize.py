"""GPU parity at the full layer size (hidden 5120, intermediate 1536, 256
experts, top-8), in the launch configuration the benchmark times.

The layer is packed on the GPU once per session; the oracle quantizes, from
the same seeded masters, every expert it needs itself and must agree
bit-for-bit on those experts.  Decode workloads (1 and 8 tokens) compare
every output; the prefill workloads (1024 and 16384 tokens) compare sampled
tokens one by one and check finiteness and magnitude everywhere.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import moe as omoe
from gpu_util import (DEFAULT_DECODE_VARIANT, DEV, bf16_bits_to_f64, compare_out, full_layer_gpu, log, oracle_experts,
                      packed_to_numpy, to_dev)
from nvfp4_weight_only_moe_amd import binding as B
from nvfp4_weight_only_moe_amd import workloads as wls

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def run_workload(cfg):
    wl = wls.WORKLOADS[cfg]
    layer = full_layer_gpu()
    xb, x = wls.activations(wl)
    lg = wls.logits(wl)
    r = B.moe_route_topk(to_dev(lg), wl.k)
    out = B.moe_w4a16_forward(to_dev(xb, torch.int16), layer["gate"], layer["up"], layer["down"], r)
    torch.cuda.synchronize()
    ids, w = oracle.route_topk(lg, wl.k)
    assert np.array_equal(r.topk_ids.cpu().numpy(), ids)
    return wl, x, ids, w, bf16_bits_to_f64(out)


def check_tokens(cfg, tokens):
    wl, x, ids, w, got = run_workload(cfg)
    experts = sorted(set(int(e) for t in tokens for e in ids[t]))
    log(f"{wl.name}: checking tokens {list(tokens)[:8]}{'...' if len(tokens) > 8 else ''} "
        f"({len(experts)} experts)")
    layer = oracle_experts(experts)
    ref = omoe.moe_forward(x, layer, ids, w, tokens=tokens)
    tokens = np.asarray(sorted(tokens))
    compare_out(got[tokens], ref[tokens], wl.name)
    assert np.all(np.isfinite(got))
    norms = np.linalg.norm(got, axis=1)
    assert np.all(norms > 0), "a token's output is exactly zero"
    return got


def test_fullsize_pack_bitexact_sampled_experts():
    layer = full_layer_gpu()
    sample = [0, 97, 255]
    ol = oracle_experts(sample)
    for name in ("gate", "up", "down"):
        codes, scales, g = packed_to_numpy(B.NVFP4Tensor(
            layer[name].codes[sample], layer[name].scales[sample], layer[name].global_scale[sample]))
        for i, e in enumerate(sample):
            assert g[i].view(np.uint32) == np.float32(ol[name][2][e]).view(np.uint32), (name, e)
            assert np.array_equal(scales[i], ol[name][1][e]), (name, e, "scales")
            assert np.array_equal(codes[i], ol[name][0][e]), (name, e, "codes")
    B.moe_w4a16_validate(layer["gate"])
    B.moe_w4a16_validate(layer["up"])
    B.moe_w4a16_validate(layer["down"])


def test_fullsize_decode_1_token():
    check_tokens(1, [0])


def test_fullsize_decode_8_tokens():
    check_tokens(2, list(range(8)))


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
@pytest.mark.parametrize("cfg", [1, 2])
def test_fullsize_route_forward_decode(cfg, variant):
    """At full size, for every decode variant: moe_w4a16_route_forward equals
    moe_route_topk followed by moe_w4a16_forward bit for bit (routing and
    output), and the output matches the oracle on sampled tokens."""
    B.moe_debug_set_decode_variant(variant)
    try:
        _route_forward_case(cfg)
    finally:
        B.moe_debug_set_decode_variant(DEFAULT_DECODE_VARIANT)


def _route_forward_case(cfg):
    wl = wls.WORKLOADS[cfg]
    layer = full_layer_gpu()
    xb, _ = wls.activations(wl)
    lg, x_d = to_dev(wls.logits(wl)), to_dev(xb, torch.int16)
    r_ref = B.moe_route_topk(lg, wl.k)
    out_ref = B.moe_w4a16_forward(x_d, layer["gate"], layer["up"], layer["down"], r_ref)
    out, r = B.moe_w4a16_route_forward(lg, x_d, layer["gate"], layer["up"], layer["down"], wl.k)
    torch.cuda.synchronize()
    for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
        assert torch.equal(getattr(r, name), getattr(r_ref, name)), name
    assert torch.equal(out, out_ref)
    log(f"{wl.name}: route_forward identical to route + forward")
    x = wls.activations(wl)[1]
    ids, w = oracle.route_topk(wls.logits(wl), wl.k)
    tokens = [0, wl.T - 1]
    experts = sorted(set(int(e) for t in tokens for e in ids[t]))
    ref = omoe.moe_forward(x, oracle_experts(experts), ids, w, tokens=tokens)
    compare_out(bf16_bits_to_f64(out)[tokens], ref[tokens], wl.name)


def test_fullsize_prefill_1024_sampled():
    check_tokens(3, [0, 511, 1023])


def test_fullsize_prefill_16384_zipf_sampled():
    wl = wls.WORKLOADS[4]
    ids, _ = oracle.route_topk(wls.logits(wl, T=64), wl.k)
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    hot = int(np.argmax(counts))
    tok_hot = int(np.nonzero((ids == hot).any(axis=1))[0][0])
    check_tokens(4, sorted({0, tok_hot, 16383}))
