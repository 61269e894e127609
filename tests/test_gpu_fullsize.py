"""GPU parity at the full layer size (hidden 5120, intermediate 1536, 256
experts, top-8), in the launch configuration the benchmark times.

The layer is packed on the GPU once per session; the oracle quantizes, from
the same seeded masters, every expert it needs itself, and the GPU-packed
codes, scales and global scale of every such expert must agree with it bit
for bit.  Decode workloads (1 and 8 tokens) compare every output; the prefill
workloads compare chosen tokens one by one -- at 1024 tokens a set that
reaches all 256 experts, at 16384 tokens one row in every 128-row tile of the
three hottest experts -- and check finiteness and magnitude everywhere.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import moe as omoe
from gpu_util import (DEV, bf16_bits_to_f64, compare_out, full_layer_gpu, log, oracle_experts,
                      oracle_forward_parallel, packed_to_numpy, to_dev)
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


def assert_packed_bitexact(experts):
    """The GPU-packed bytes of every listed expert equal the oracle's."""
    gpu = full_layer_gpu()
    ol = oracle_experts(experts)
    idx = torch.as_tensor(sorted(int(e) for e in experts), device=DEV)
    for name in ("gate", "up", "down"):
        codes, scales, g = packed_to_numpy(B.NVFP4Tensor(
            gpu[name].codes[idx].contiguous(), gpu[name].scales[idx].contiguous(),
            gpu[name].global_scale[idx].contiguous()))
        for i, e in enumerate(idx.tolist()):
            assert g[i].view(np.uint32) == np.float32(ol[name][2][e]).view(np.uint32), (name, e, "global")
            assert np.array_equal(scales[i], ol[name][1][e]), (name, e, "scales")
            assert np.array_equal(codes[i], ol[name][0][e]), (name, e, "codes")
    log(f"packed bytes bit-exact on {len(idx)} experts x 3 projections")


def check_tokens(cfg, tokens):
    wl, x, ids, w, got = run_workload(cfg)
    experts = sorted(set(int(e) for t in tokens for e in ids[t]))
    log(f"{wl.name}: checking {len(tokens)} tokens {list(tokens)[:8]}{'...' if len(tokens) > 8 else ''} "
        f"({len(experts)} experts)")
    layer = oracle_experts(experts)
    assert_packed_bitexact(experts)
    ref = oracle_forward_parallel(x, layer, ids, w, tokens)
    tokens = np.asarray(sorted(tokens))
    compare_out(got[tokens], ref[tokens], wl.name)
    assert np.all(np.isfinite(got))
    norms = np.linalg.norm(got, axis=1)
    assert np.all(norms > 0), "a token's output is exactly zero"
    return got


def test_fullsize_pack_bitexact_sampled_experts():
    assert_packed_bitexact([0, 97, 255])
    layer = full_layer_gpu()
    flag = torch.zeros((4,), dtype=torch.int32, device=DEV)
    for name in ("gate", "up", "down"):
        B.moe_w4a16_validate(layer[name], flag)


def test_fullsize_decode_1_token():
    check_tokens(1, [0])


def test_fullsize_decode_8_tokens():
    check_tokens(2, list(range(8)))


@pytest.mark.parametrize("cfg", [1, 2])
def test_fullsize_route_forward_decode(cfg):
    """At full size, moe_w4a16_route_forward (one token: the route inside the
    gate/up kernel) equals moe_route_topk followed by moe_w4a16_forward bit
    for bit (routing and output), and the output matches the oracle."""
    _route_forward_case(cfg)


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
    tokens = list(range(wl.T))
    experts = sorted(set(int(e) for t in tokens for e in ids[t]))
    assert_packed_bitexact(experts)
    ref = oracle_forward_parallel(x, oracle_experts(experts), ids, w, tokens)
    compare_out(bf16_bits_to_f64(out)[tokens], ref[tokens], wl.name)


def covering_tokens(ids, E, at_least):
    """Tokens chosen greedily until every expert that any token touches is
    reached (each pick adds the most unreached experts; ties to the lower
    token), then topped up with evenly spaced tokens to `at_least`."""
    T = ids.shape[0]
    reached = np.zeros(E, bool)
    want = np.zeros(E, bool)
    want[np.unique(ids)] = True
    chosen = []
    while (want & ~reached).any():
        gain = (~reached[ids]).sum(axis=1)
        gain[chosen] = -1
        t = int(np.argmax(gain))
        chosen.append(t)
        reached[ids[t]] = True
    for t in np.linspace(0, T - 1, at_least).astype(int):
        if len(chosen) >= at_least:
            break
        if int(t) not in chosen:
            chosen.append(int(t))
    return sorted(chosen)


def test_fullsize_prefill_1024_all_experts():
    wl = wls.WORKLOADS[3]
    ids, _ = oracle.route_topk(wls.logits(wl), wl.k)
    tokens = covering_tokens(ids, wl.E, 64)
    assert len(set(ids[tokens].ravel())) == wl.E
    assert len(tokens) >= 64
    check_tokens(3, tokens)


def test_fullsize_prefill_16384_zipf_hot_expert_tiles():
    """One row in every 128-row tile (the LDS-pipelined kernel's row tile at
    this size) of the three hottest experts, at an offset inside the tile
    that moves from tile to tile, plus the first and last tokens."""
    wl = wls.WORKLOADS[4]
    ids, _ = oracle.route_topk(wls.logits(wl), wl.k)
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    hottest = np.argsort(-counts, kind="stable")[:3]
    tokens = {0, wl.T - 1}
    for rank, e in enumerate(hottest):
        rows = np.nonzero((ids == e).any(axis=1))[0]      # the expert's rows in sorted order
        assert rows.size == counts[e]
        for m in range((rows.size + 127) // 128):
            r = min(m * 128 + (37 * m + 11 * rank) % 128, rows.size - 1)
            tokens.add(int(rows[r]))
        log(f"expert {int(e)}: {rows.size} rows, {(rows.size + 127) // 128} row tiles")
    assert counts[hottest[0]] > 8 * 128 * 2                  # several groups of 8 row tiles
    check_tokens(4, sorted(tokens))
