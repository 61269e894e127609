"""GPU parity: the layer forward against the oracle on small seeded problems
(decode path: T <= 8 with H % 1024 == 0 and I % 512 == 0; grouped-GEMM path
otherwise), ragged and skewed routing, experts long enough to span several
scheduling groups of row tiles, edge cases, determinism.  Every output,
routing array and workspace is allocated between guard bands that must stay
untouched (gpu_util.Guarded)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, Problem, bf16_bits_to_f64, compare_out, guarded_forward, log, to_dev
from nvfp4_weight_only_moe_amd import binding as B
from nvfp4_weight_only_moe_amd import workloads as wls

pytestmark = pytest.mark.gpu


def run_and_compare(p, where, fused=False):
    out, r, _ = p.run_gpu(fused)
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
@pytest.mark.parametrize("fused", [False, True])
def test_random_shapes(T, H, I, E, k, seed, fused):
    run_and_compare(Problem(T, H, I, E, k, seed), f"T{T}-H{H}-I{I}-E{E}-k{k}", fused)


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
        ws.fill_(0xAB)          # the workspace needs no initialisation
        B.moe_w4a16_forward(xb, gate, up, down, other)      # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"


# ------------------------------------------------------------------ route + forward in one call
DECODE_CASES = [
    (1, 1024, 512, 8, 2, 70),
    (1, 2048, 1536, 8, 6, 71),
    (4, 2048, 1024, 32, 8, 72),
    (8, 1024, 1536, 8, 8, 73),       # k == E
    (8, 3072, 512, 300, 8, 74),      # E > 256: five logits per lane in the top-k
    (1, 8192, 2048, 4, 2, 76),       # the largest decode shape: H = 8192, I = 2048
    (8, 8192, 2048, 4, 3, 77),
]


@pytest.mark.parametrize("T,H,I,E,k,seed", DECODE_CASES + [(40, 512, 256, 16, 4, 75)])
def test_route_forward_matches_route_then_forward(T, H, I, E, k, seed):
    """moe_w4a16_route_forward stores exactly moe_route_topk's outputs and
    exactly moe_w4a16_forward's result (with one token the route runs inside
    the gate/up kernel), and matches the oracle."""
    p = Problem(T, H, I, E, k, seed)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    log(f"route_forward T{T} H{H} I{I} E{E} k{k}")
    out_ref, r_ref = guarded_forward(xb, gate, up, down, lg, k, fused=False)
    out, r = guarded_forward(xb, gate, up, down, lg, k, fused=True)
    for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
        assert torch.equal(getattr(r, name), getattr(r_ref, name)), name
    assert np.array_equal(r.topk_ids.cpu().numpy(), p.ids)
    assert torch.equal(out, out_ref)
    compare_out(bf16_bits_to_f64(out), p.reference(), f"route_forward-T{T}")


@pytest.mark.parametrize("E", [64, 256])
def test_route_forward_ties(E):
    """One token whose logits hold many exact ties (integers): the routing
    computed inside the gate/up kernel picks the same experts, in the same
    order, as moe_route_topk and the oracle."""
    T, H, I, k = 1, 1024, 512, 8
    lg_np = np.random.default_rng(E).integers(-2, 3, size=(T, E)).astype(np.float32)
    lg_np[0, 3] = -0.0
    p = Problem(T, H, I, E, k, 300 + E, logits=lg_np)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    out_ref, r_ref = guarded_forward(xb, gate, up, down, lg, k, fused=False)
    out, r = guarded_forward(xb, gate, up, down, lg, k, fused=True)
    for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
        assert torch.equal(getattr(r, name), getattr(r_ref, name)), name
    assert np.array_equal(r.topk_ids.cpu().numpy(), p.ids)
    assert torch.equal(out, out_ref)


def test_workspace_reused_across_problems():
    """One workspace serves consecutive calls with different inputs, routings
    and shapes, and garbage left in it between calls changes nothing: no
    call reads a value it did not write in the same call."""
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
    for rnd, fill in enumerate((0x00, 0x5A, 0xFF)):
        ws.fill_(fill)
        for p, packed, fresh in probs:
            out, _ = B.moe_w4a16_route_forward(to_dev(p.logits), to_dev(p.xb, torch.int16), *packed, p.k, ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(out, fresh), f"round {rnd} T{p.T} H{p.H}"


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
    (300, 512, 384, 4, 2, 98),       # 128-row tiles, I % 256 != 0: down without the LDS scale blocks
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
            out, _ = guarded_forward(xb, gate, up, down, lg, k, fused=True)
            got = bf16_bits_to_f64(out)
            compare_out(got, ref, f"prefill variant {v} T{T}")
            outs.append(got)
    finally:
        B.moe_debug_set_prefill_variant(2)
    for v in (1, 2):
        compare_out(outs[v], outs[0], f"prefill variant {v} vs 0")


# Experts long enough that the grouped GEMMs' tile numbering (an expert's row
# tiles in scheduling groups of 8 x all column tiles, then a tail group) runs
# through whole groups, every offset inside a group and the tail: one expert
# is made hot (+40 on its logit), so it holds every token.  Gate/up and down
# both have two column tiles.  Per case: (T, H, I, E, k, seed, register-staged
# row tile that variant 0 picks by the mean rows per touched expert).
LONG_EXPERT_CASES = [
    (2200, 1024, 512, 4, 2, 110, 128),     # 17+ tiles of 128: 2 groups + tail (both kernels)
    (2100, 512, 512, 72, 2, 111, 64),      # 33 tiles of 64: 4 groups + tail; 16+ of 128
    (1500, 512, 512, 200, 2, 112, 32),     # 47 tiles of 32: 5 groups + tail; 11+ of 128
]


@pytest.mark.parametrize("T,H,I,E,k,seed,bm", LONG_EXPERT_CASES)
def test_prefill_long_expert_every_tile(T, H, I, E, k, seed, bm):
    """Every token compared against the oracle, for every grouped-GEMM kernel
    choice, on experts that span several groups of 8 row tiles."""
    r = np.random.default_rng(seed)
    lg_np = r.standard_normal((T, E)).astype(np.float32)
    hot = 1
    lg_np[:, hot] += 40.0
    p = Problem(T, H, I, E, k, seed, logits=lg_np)
    slots = T * k
    avg = slots // min(E, slots)
    assert (avg <= 16) == (bm == 32) and (16 < avg <= 64) == (bm == 64), "variant 0 row tile"
    counts = np.bincount(p.ids.ravel(), minlength=E)
    assert counts[hot] == T and counts[hot] >= 2 * 8 * bm + 1, counts[hot]
    assert counts[hot] >= 8 * 128 + 1                          # the pipelined kernel's 128-row tiles too
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    ref = p.reference()
    try:
        for v in (0, 1, 2):
            B.moe_debug_set_prefill_variant(v)
            out, _ = guarded_forward(xb, gate, up, down, lg, k, fused=True)
            got = bf16_bits_to_f64(out)
            compare_out(got, ref, f"long expert T{T} E{E} variant {v}")
            # rows of the hot expert, row tile by row tile: each tile's worst row
            err = np.abs(got - ref).max(axis=1) / np.abs(ref).max()
            tiles = [err[i:i + bm].max() for i in range(0, T, bm)]
            assert max(tiles) <= 1e-2, (v, int(np.argmax(tiles)))
    finally:
        B.moe_debug_set_prefill_variant(2)


@pytest.mark.parametrize("E,k,ties", [(300, 8, False), (1024, 32, False), (1024, 8, True), (64, 32, True),
                                      (256, 1, False), (9, 8, True)])
def test_one_token_in_kernel_route(E, k, ties):
    """One token routed inside the gate/up kernel (threshold selection): every
    routing output equals moe_route_topk's and the oracle's, and the layer
    output equals the two-call path's, bit for bit -- wide routers (up to
    1024 experts, 16 logits per lane), k up to 64, exact ties.  The weights
    come from the GPU quantizer (no layer oracle needed for equality)."""
    H, I = 1024, 512
    g = torch.Generator(device=DEV).manual_seed(E * 100 + k)
    stacks = [B.moe_w4a16_quantize_pack(0.02 * torch.randn((E,) + s, device=DEV, generator=g))
              for s in ((I, H), (I, H), (H, I))]
    r = np.random.default_rng(E + k)
    lg_np = (r.integers(-3, 4, size=(1, E)) if ties else r.standard_normal((1, E))).astype(np.float32)
    if ties:
        lg_np[0, :: 7] = -0.0
    x = to_dev(wls.to_bf16_bits(r.standard_normal((1, H)).astype(np.float32)).view(np.int16))
    lg = to_dev(lg_np)
    out_ref, r_ref = guarded_forward(x, *stacks, lg, k, fused=False)
    out, r_got = guarded_forward(x, *stacks, lg, k, fused=True)
    for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
        assert torch.equal(getattr(r_got, name), getattr(r_ref, name)), name
    ids, w = oracle.route_topk(lg_np, k)
    assert np.array_equal(r_got.topk_ids.cpu().numpy(), ids)
    assert np.max(np.abs(r_got.topk_w.cpu().numpy() - w)) <= 1e-6
    assert torch.equal(out, out_ref)
