"""GPU parity of the W4A4 NVFP4 variant (activations quantized to NVFP4 with a
static input scale) against the oracle (oracle/w4a4.py): the activation
codes and scales bit-exact, the layer output within the forward's bar, bad
input scales refused before any work.  Through the C ABI, with guard bands
around every buffer the library writes."""
import numpy as np
import pytest
import torch

import oracle
from oracle import w4a4 as ow4
from gpu_util import (DEV, Guarded, Problem, bf16_bits_to_f64, check_guards, compare_out, full_layer_gpu,
                      guarded_routing, log, oracle_experts, to_dev)
from nvfp4_weight_only_moe_amd import binding as B
from nvfp4_weight_only_moe_amd import workloads as wls

pytestmark = pytest.mark.gpu

SX, SH = wls.W4A4_INPUT_SCALES


def act_cases():
    r = np.random.default_rng(7)
    x = r.standard_normal((37, 512)).astype(np.float32)
    x[0, :16] = 0.0
    x[1, :16] = -0.0
    x[2, 16:32] *= np.float32(1e-5)              # small-amax group: subnormal or zero scale
    x[3, 40] = 80.0                              # saturating group
    x[4, :] = np.float32(6 * SX) * np.float32(448)   # exactly the largest code at the largest scale
    return x


@pytest.mark.parametrize("scale", [SX, 1.0, 2.0 ** -12])
def test_activation_quantization_bitexact(scale):
    x = act_cases()
    xb = wls.to_bf16_bits(x)
    xv = wls.bf16_bits_to_f32(xb)
    codes = Guarded((x.shape[0], x.shape[1] // 2), torch.uint8)
    scales = Guarded((x.shape[0], x.shape[1] // 16), torch.uint8)
    B.moe_nvfp4_quantize_activations(to_dev(xb.view(np.int16)), scale, codes=codes.t, scales=scales.t)
    torch.cuda.synchronize()
    codes.check("codes")
    scales.check("scales")
    oc, os_ = ow4.quantize_activations(xv, scale)
    assert np.array_equal(scales.t.cpu().numpy(), os_)
    assert np.array_equal(codes.t.cpu().numpy(), oc)


@pytest.mark.parametrize("bad", [0.0, -0.0, -1.0, float("nan"), float("inf")])
def test_bad_input_scales_refused(bad):
    p = Problem(4, 256, 128, 8, 2, 500)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    r = B.moe_route_topk(to_dev(p.logits), 2)
    xb = to_dev(p.xb, torch.int16)
    want = "MOE_ERR_NONFINITE" if bad != bad or bad in (float("inf"),) else "MOE_ERR_BAD_SCALE"
    for sx, sh in ((bad, SH), (SX, bad)):
        out = torch.full((4, 256), 7, dtype=torch.int16, device=DEV)
        with pytest.raises(B.MoeError) as err:
            B.moe_w4a4_forward(xb, gate, up, down, r, sx, sh, out=out)
        assert B.STATUS[err.value.status] == want
        torch.cuda.synchronize()
        assert bool((out == 7).all()), "a refused call wrote its output"
    with pytest.raises(B.MoeError):
        B.moe_nvfp4_quantize_activations(xb, bad)
    with pytest.raises(ValueError):
        B.moe_w4a4_forward(xb, gate, up, down, r, None, SH)
    # T = 0 is still refused with a bad scale
    r0 = B.moe_route_topk(to_dev(p.logits[:0]), 2)
    with pytest.raises(B.MoeError):
        B.moe_w4a4_forward(xb[:0], gate, up, down, r0, bad, SH)


def run_w4a4(p, sx, sh):
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    T, H, E, k = p.T, p.H, p.E, p.k
    r, parts = guarded_routing(T, E, k)
    B.moe_route_topk(to_dev(p.logits), k, out=r)
    parts["out"] = Guarded((T, H), torch.int16)
    parts["ws"] = Guarded((max(B.moe_w4a4_workspace_size(T, H, p.I, E, k), 16),), torch.uint8)
    B.moe_w4a4_forward(to_dev(p.xb, torch.int16), gate, up, down, r, sx, sh, out=parts["out"].t, ws=parts["ws"].t)
    torch.cuda.synchronize()
    check_guards(parts, f"w4a4 T{T} H{H} I{p.I} E{E} k{k}")
    return bf16_bits_to_f64(parts["out"].t), r


W4A4_CASES = [
    (1, 1024, 512, 8, 2, 601),        # decode kernels
    (8, 2048, 1024, 32, 8, 602),
    (33, 256, 128, 8, 2, 603),        # grouped GEMM, 32-row tiles
    (100, 512, 384, 16, 4, 604),      # 64-row tiles, ragged
    (700, 512, 256, 8, 4, 605),       # LDS-pipelined kernels (350 rows per expert)
]


@pytest.mark.parametrize("T,H,I,E,k,seed", W4A4_CASES)
def test_w4a4_forward_parity(T, H, I, E, k, seed):
    p = Problem(T, H, I, E, k, seed)
    # calibration-like scales for these shapes: |x| up to ~5, h up to ~3 at H <= 2048
    sx, sh = np.float32(5.0 / 2688.0), np.float32(4.0 / 2688.0)
    got, r = run_w4a4(p, sx, sh)
    assert np.array_equal(r.topk_ids.cpu().numpy(), p.ids)
    ref = ow4.moe_forward_w4a4(p.x, p.layer, p.ids, p.w, sx, sh)
    compare_out(got, ref, f"w4a4 T{T} H{H} I{I} E{E} k{k}")
    # clearly not the W4A16 result: the activations were quantized
    w16 = p.reference()
    d = np.linalg.norm(got - w16) / np.linalg.norm(w16)
    log(f"w4a4 T{T}: relative difference to the W4A16 oracle {d:.3e}")
    assert d > 5e-3


@pytest.mark.parametrize("T,H,I,E,k,seed", [
    (1, 1024, 512, 16, 8, 620),       # one token: the gate/up kernel routes itself
    (1, 2048, 1024, 12, 3, 621),      # one token, another shape
    (8, 1024, 512, 16, 4, 622),       # decode kernels after the route launch
    (100, 512, 256, 16, 4, 623),      # grouped GEMMs after the route launch
])
def test_w4a4_route_forward_equals_route_then_forward(T, H, I, E, k, seed):
    """moe_w4a4_route_forward stores exactly moe_route_topk's routing and
    returns exactly moe_w4a4_forward's output on it, bit for bit."""
    p = Problem(T, H, I, E, k, seed)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    sx, sh = np.float32(5.0 / 2688.0), np.float32(4.0 / 2688.0)
    xb, lg = to_dev(p.xb, torch.int16), to_dev(p.logits)
    r_ref = B.moe_route_topk(lg, k)
    ref = B.moe_w4a4_forward(xb, gate, up, down, r_ref, sx, sh)
    r, parts = guarded_routing(T, E, k)
    parts["out"] = Guarded((T, H), torch.int16)
    parts["ws"] = Guarded((max(B.moe_w4a4_workspace_size(T, H, I, E, k), 16),), torch.uint8)
    B.moe_w4a4_route_forward(lg, xb, gate, up, down, k, sx, sh, routing=r, out=parts["out"].t, ws=parts["ws"].t)
    torch.cuda.synchronize()
    check_guards(parts, f"w4a4 route_forward T{T} E{E} k{k}")
    for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
        assert torch.equal(getattr(r, name), getattr(r_ref, name)), (T, name)
    assert torch.equal(parts["out"].t, ref), T
    compare_out(bf16_bits_to_f64(ref), ow4.moe_forward_w4a4(p.x, p.layer, p.ids, p.w, sx, sh),
                f"w4a4 route_forward T{T} H{H} E{E} k{k}")


@pytest.mark.parametrize("variant", [0, 1])
def test_w4a4_long_expert_every_tile(variant):
    T, H, I, E, k, seed = 2200, 1024, 512, 4, 2, 610
    r = np.random.default_rng(seed)
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg[:, 2] += 40.0
    p = Problem(T, H, I, E, k, seed, logits=lg)
    sx, sh = np.float32(5.0 / 2688.0), np.float32(4.0 / 2688.0)
    try:
        B.moe_debug_set_prefill_variant(variant)
        got, _ = run_w4a4(p, sx, sh)
    finally:
        B.moe_debug_set_prefill_variant(2)
    compare_out(got, ow4.moe_forward_w4a4(p.x, p.layer, p.ids, p.w, sx, sh), f"w4a4 long expert variant {variant}")


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_w4a4_fullsize(cfg):
    """The full-size layer (configs 1-3) with the workloads' input scales;
    every token at decode, a covering sample of 24 tokens at 1024."""
    wl = wls.WORKLOADS[cfg]
    layer = full_layer_gpu()
    xb, x = wls.activations(wl)
    lg = wls.logits(wl)
    r = B.moe_route_topk(to_dev(lg), wl.k)
    out = B.moe_w4a4_forward(to_dev(xb, torch.int16), layer["gate"], layer["up"], layer["down"], r, SX, SH)
    torch.cuda.synchronize()
    ids, w = oracle.route_topk(lg, wl.k)
    tokens = list(range(wl.T)) if wl.T <= 8 else list(range(0, wl.T, wl.T // 24))[:24]
    experts = sorted(set(int(e) for t in tokens for e in ids[t]))
    ref = ow4.moe_forward_w4a4(x, oracle_experts(experts), ids, w, SX, SH, tokens=tokens)
    got = bf16_bits_to_f64(out)
    compare_out(got[tokens], ref[tokens], f"w4a4 {wl.name}")
