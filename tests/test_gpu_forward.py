"""GPU parity: the layer forward against the oracle on small seeded problems
(decode path: T <= 8 with H % 1024 == 0 and I % 512 == 0; grouped-GEMM path
otherwise), ragged and skewed routing, edge cases, determinism."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEFAULT_DECODE_VARIANT, DEV, Problem, bf16_bits_to_f64, compare_out, log, to_dev
from nvfp4_weight_only_moe_amd import binding as B
from nvfp4_weight_only_moe_amd import workloads as wls

pytestmark = pytest.mark.gpu


def run_and_compare(p, where):
    out, r, _ = p.run_gpu()
    assert np.array_equal(r.topk_ids.cpu().numpy(), p.ids)
    got = bf16_bits_to_f64(out)
    ref = p.reference()
    compare_out(got, ref, where)
    # the diagnostic oracle rounds h to bf16 like the device: much closer
    tight = p.reference(round_h_bf16=True)
    rel = np.linalg.norm(got - tight) / np.linalg.norm(tight)
    log(f"{where}: rel_fro vs bf16-h oracle {rel:.3e}")
    return got


def test_tiny_workload():
    wl = wls.WORKLOADS[0]
    ms = [wls.masters(wl, p) for p in (wls.GATE, wls.UP, wls.DOWN)]
    xb, x = wls.activations(wl)
    lg = wls.logits(wl)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in ms)
    r = B.moe_route_topk(to_dev(lg), wl.k)
    out = B.moe_w4a16_forward(to_dev(xb, torch.int16), gate, up, down, r)
    torch.cuda.synchronize()
    layer = {n: oracle.quantize_layer(m) for n, m in zip(("gate", "up", "down"), ms)}
    ids, w = oracle.route_topk(lg, wl.k)
    ref = oracle.moe_forward(x, layer, ids, w)
    compare_out(bf16_bits_to_f64(out), ref, wl.name)


@pytest.mark.parametrize("T,H,I,E,k,seed", [
    (1, 1024, 512, 8, 2, 1),       # decode path
    (3, 1024, 512, 16, 4, 2),
    (8, 2048, 1024, 32, 8, 3),
    (8, 1024, 1536, 8, 8, 4),      # k == E: every expert touched by every token
    (9, 1024, 512, 16, 2, 5),      # just past the decode path
    (33, 256, 128, 8, 2, 6),       # grouped GEMM, 32-row tiles
    (100, 512, 384, 16, 4, 7),     # 64-row tiles, ragged
    (257, 256, 256, 4, 2, 8),      # 128-row tiles, several row tiles per expert
    (40, 768, 256, 1, 1, 9),       # E = 1, k = 1
])
def test_random_shapes(T, H, I, E, k, seed):
    run_and_compare(Problem(T, H, I, E, k, seed), f"T{T}-H{H}-I{I}-E{E}-k{k}")


@pytest.mark.parametrize("T,H,I", [(6, 1024, 512), (300, 256, 128)])
def test_all_tokens_on_one_expert(T, H, I):
    E, k = 16, 2
    r = np.random.default_rng(T)
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg[:, 11] += 40.0
    run_and_compare(Problem(T, H, I, E, k, 20 + T, logits=lg), f"skew-T{T}")


def test_zero_tokens_is_noop():
    p = Problem(4, 256, 128, 8, 2, 30)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    r = B.moe_route_topk(to_dev(p.logits[:0]), 2)
    out = torch.full((0, 256), 7, dtype=torch.int16, device=DEV)
    B.moe_w4a16_forward(torch.zeros((0, 256), dtype=torch.int16, device=DEV), gate, up, down, r, out=out)
    torch.cuda.synchronize()


def test_zero_input_gives_zero_output():
    p = Problem(5, 256, 128, 8, 2, 31)
    p.xb[:] = 0
    out, _, _ = p.run_gpu()
    assert not bf16_bits_to_f64(out).any()


@pytest.mark.parametrize("T,H,I", [(8, 1024, 512), (120, 512, 256)])
def test_deterministic(T, H, I):
    p = Problem(T, H, I, 16, 4, 40)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    r = B.moe_route_topk(to_dev(p.logits), 4)
    xb = to_dev(p.xb, torch.int16)
    a = B.moe_w4a16_forward(xb, gate, up, down, r)
    b = B.moe_w4a16_forward(xb, gate, up, down, r)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_magnitude_not_correlation_only():
    """A layer whose global scales are scaled by 25 keeps cosine ~1 but must
    fail the output bar -- the check that catches a wrong scale
    ('GLM-5.3-Flash on Blackwell': a 25x magnitude error at cosine 0.996)."""
    p = Problem(6, 1024, 512, 8, 2, 50)
    out, r, (gate, up, down) = p.run_gpu()
    down.global_scale.mul_(25.0)
    bad = B.moe_w4a16_forward(to_dev(p.xb, torch.int16), gate, up, down, r)
    torch.cuda.synchronize()
    with pytest.raises(AssertionError):
        compare_out(bf16_bits_to_f64(bad), p.reference(), "scaled-by-25")


@pytest.mark.parametrize("T,H,I", [(8, 1024, 512), (100, 512, 256)])
def test_hip_graph_replay_matches_eager(T, H, I):
    """route + forward captured in a HIP graph: every replay, with unrelated
    eager work between replays, reproduces the eager output bit for bit."""
    E, k = 16, 4
    p = Problem(T, H, I, E, k, 60 + T)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    route = B.Routing.empty(T, E, k, DEV)
    out = torch.empty((T, H), dtype=torch.int16, device=DEV)
    ws = B.forward_workspace(T, H, I, E, k, DEV)

    def step():
        B.moe_route_topk(lg, k, out=route)
        B.moe_w4a16_forward(xb, gate, up, down, route, out=out, ws=ws)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = B.moe_route_topk(to_dev(p.logits[::-1].copy()), k)
    for i in range(4):
        out.fill_(i + 1)
        ws[256:].fill_(0xAB)    # everything but the sync words, which calls keep at zero
        B.moe_w4a16_forward(xb, gate, up, down, other)      # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"


# ------------------------------------------------------------------ route + forward in one call
@pytest.fixture
def decode_variant(request):
    """Select the decode-shape kernels (moe_debug_set_decode_variant) for one
    test; the default is restored afterwards."""
    B.moe_debug_set_decode_variant(request.param)
    yield request.param
    B.moe_debug_set_decode_variant(DEFAULT_DECODE_VARIANT)


DECODE_CASES = [
    (1, 1024, 512, 8, 2, 70),
    (1, 2048, 1536, 8, 6, 71),
    (4, 2048, 1024, 32, 8, 72),
    (8, 1024, 1536, 8, 8, 73),       # k == E
    (8, 3072, 512, 300, 8, 74),      # E > 256: five logits per lane in the top-k
]


@pytest.mark.parametrize("decode_variant", [0, 1, 2, 3], indirect=True)
@pytest.mark.parametrize("T,H,I,E,k,seed", DECODE_CASES + [(40, 512, 256, 16, 4, 75)])
def test_route_forward_matches_route_then_forward(T, H, I, E, k, seed, decode_variant):
    """moe_w4a16_route_forward stores exactly moe_route_topk's outputs and
    exactly moe_w4a16_forward's result (with variants 1 and 3 the route runs
    inside the layer's kernels), for every decode variant, and matches the
    oracle."""
    p = Problem(T, H, I, E, k, seed)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    log(f"route_forward T{T} H{H} I{I} E{E} k{k} decode variant {decode_variant}")
    r_ref = B.moe_route_topk(lg, k)
    out_ref = B.moe_w4a16_forward(xb, gate, up, down, r_ref)
    out, r = B.moe_w4a16_route_forward(lg, xb, gate, up, down, k)
    torch.cuda.synchronize()
    for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
        assert torch.equal(getattr(r, name), getattr(r_ref, name)), name
    assert np.array_equal(r.topk_ids.cpu().numpy(), p.ids)
    assert torch.equal(out, out_ref)
    compare_out(bf16_bits_to_f64(out), p.reference(), f"route_forward-T{T}")


@pytest.mark.parametrize("decode_variant", [0, 1, 3], indirect=True)
@pytest.mark.parametrize("E", [64, 256])
def test_route_forward_ties(E, decode_variant):
    """One token whose logits hold many exact ties (integers): the routing
    computed inside the layer's kernels picks the same experts, in the same
    order, as moe_route_topk and the oracle."""
    T, H, I, k = 1, 1024, 512, 8
    lg_np = np.random.default_rng(E).integers(-2, 3, size=(T, E)).astype(np.float32)
    lg_np[0, 3] = -0.0
    p = Problem(T, H, I, E, k, 300 + E, logits=lg_np)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    r_ref = B.moe_route_topk(lg, k)
    out_ref = B.moe_w4a16_forward(xb, gate, up, down, r_ref)
    out, r = B.moe_w4a16_route_forward(lg, xb, gate, up, down, k)
    torch.cuda.synchronize()
    for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
        assert torch.equal(getattr(r, name), getattr(r_ref, name)), name
    assert np.array_equal(r.topk_ids.cpu().numpy(), p.ids)
    assert torch.equal(out, out_ref)


@pytest.mark.parametrize("decode_variant", [1], indirect=True)
@pytest.mark.parametrize("T,H,I,E,k,seed", DECODE_CASES[:3])
def test_decode_local_h_path_is_bit_identical(T, H, I, E, k, seed, decode_variant):
    """With the hand-off wait limit at 0 every workgroup computes all of h
    itself (the path taken when the grid is not fully resident); the result
    is bit-identical to the normal hand-off."""
    p = Problem(T, H, I, E, k, seed)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    out_ref, _ = B.moe_w4a16_route_forward(lg, xb, gate, up, down, k)
    torch.cuda.synchronize()
    ws = B.forward_workspace(T, H, I, E, k, DEV)
    try:
        B.moe_debug_set_decode_wait_limit(0)
        outs = [B.moe_w4a16_route_forward(lg, xb, gate, up, down, k, ws=ws)[0] for _ in range(2)]
        torch.cuda.synchronize()
    finally:
        B.moe_debug_set_decode_wait_limit(1 << 20)
    for o in outs:
        assert torch.equal(o, out_ref)
    # the workspace is still good for the normal path afterwards
    again, _ = B.moe_w4a16_route_forward(lg, xb, gate, up, down, k, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(again, out_ref)


@pytest.mark.parametrize("decode_variant", [1, 2, 3], indirect=True)
def test_workspace_reused_across_problems(decode_variant):
    """One workspace serves consecutive calls with different inputs, routings
    and shapes: no call reads another call's intermediate values, and
    moe_w4a16_workspace_init restores a workspace whose sync words were
    overwritten."""
    cases = [(1, 1024, 512, 16, 4, 80), (8, 1024, 512, 16, 4, 81), (3, 2048, 512, 16, 4, 82),
             (1, 1024, 512, 16, 4, 83), (50, 1024, 512, 16, 4, 84), (2, 1024, 512, 16, 4, 85)]
    ws = B.forward_workspace(50, 2048, 512, 16, 4, DEV)
    probs = []
    for T, H, I, E, k, seed in cases:
        p = Problem(T, H, I, E, k, seed)
        packed = [B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms]
        fresh, _ = B.moe_w4a16_route_forward(to_dev(p.logits), to_dev(p.xb, torch.int16), *packed, k)
        probs.append((p, packed, fresh))
    torch.cuda.synchronize()
    for rnd in range(2):
        for p, packed, fresh in probs:
            out, _ = B.moe_w4a16_route_forward(to_dev(p.logits), to_dev(p.xb, torch.int16), *packed, p.k, ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(out, fresh), f"round {rnd} T{p.T} H{p.H}"
        ws.fill_(0x5A)
        B.moe_w4a16_workspace_init(ws)


@pytest.mark.parametrize("T,H,I,E,k,seed", DECODE_CASES)
def test_decode_variants_agree(T, H, I, E, k, seed):
    """The decode-shape kernel sets each match the oracle, and agree with
    one another to the forward's tolerance."""
    p = Problem(T, H, I, E, k, seed)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    ref = p.reference()
    outs = []
    try:
        for v in (0, 1, 2, 3):
            B.moe_debug_set_decode_variant(v)
            out, _ = B.moe_w4a16_route_forward(lg, xb, gate, up, down, k)
            torch.cuda.synchronize()
            got = bf16_bits_to_f64(out)
            compare_out(got, ref, f"variant {v} T{T}")
            outs.append(got)
    finally:
        B.moe_debug_set_decode_variant(DEFAULT_DECODE_VARIANT)
    for v in (1, 2, 3):
        compare_out(outs[v], outs[0], f"variant {v} vs 0")


PREFILL_CASES = [
    # the LDS-pipelined kernels take H % 512 == 0 and I % 256 == 0
    (33, 512, 256, 8, 2, 90),        # one short row tile per expert, K = 256 (four stages)
    (100, 1024, 512, 16, 4, 91),     # ragged row tiles
    (257, 512, 256, 4, 2, 92),       # several row tiles per expert
    (300, 1024, 512, 8, 8, 93),      # k == E
    (40, 1024, 256, 1, 1, 94),       # E = 1, k = 1
    (600, 2048, 1536, 8, 4, 95),     # longer K: the ring runs across tile boundaries
    (100, 512, 384, 16, 4, 96),      # I % 256 != 0: the register-staged kernels in every variant
    (700, 512, 256, 8, 4, 97),       # 350 rows per expert: variant 2 takes the LDS-pipelined kernels
]


@pytest.mark.parametrize("T,H,I,E,k,seed", PREFILL_CASES)
def test_prefill_variants_agree(T, H, I, E, k, seed):
    """Every grouped-GEMM kernel choice matches the oracle and the others."""
    p = Problem(T, H, I, E, k, seed)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    ref = p.reference()
    outs = []
    try:
        for v in (0, 1, 2):
            B.moe_debug_set_prefill_variant(v)
            log(f"prefill variant {v} T{T} H{H} I{I} E{E} k{k}")
            out, _ = B.moe_w4a16_route_forward(lg, xb, gate, up, down, k)
            torch.cuda.synchronize()
            got = bf16_bits_to_f64(out)
            compare_out(got, ref, f"prefill variant {v} T{T}")
            outs.append(got)
    finally:
        B.moe_debug_set_prefill_variant(2)
    for v in (1, 2):
        compare_out(outs[v], outs[0], f"prefill variant {v} vs 0")
