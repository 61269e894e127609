"""GPU parity of the router logits (moe_router_logits) against the oracle.

Tolerance, derived from the arithmetic: the products of two bf16 values are
exact in fp32, so the only error is the fp32 summation of H terms; in any
order it is at most gamma_H * sum_i |x_i w_i| with gamma_n = n u / (1 - n u)
(u = 2^-24; taken as 2^-23 to cover an accumulator that truncates).  The
bound is per element, on the seeded inputs of the workload generators; the
oracle sums in fp64."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_weight_only_moe_amd import binding as B
from nvfp4_weight_only_moe_amd import workloads as wls
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def bound(xa, wa):
    H = xa.shape[1]
    u = 2.0 ** -23
    gamma = H * u / (1 - H * u)
    return gamma * oracle.router_logits(np.abs(xa), np.abs(wa)) + 1e-30


def run(T, H, E, seed):
    xb, x, wb, w = wls.router_problem(seed, T, H, E)
    got = B.moe_router_logits(to_dev(xb, torch.int16), to_dev(wb, torch.int16))
    torch.cuda.synchronize()
    return got.cpu().numpy().astype(np.float64), oracle.router_logits(x, w), bound(x, w)


CASES = [
    # 1-8 tokens: the GEMV
    (1, 5120, 256, 1), (2, 1024, 64, 2), (5, 2048, 100, 3), (8, 5120, 256, 4), (3, 64, 1, 5), (7, 192, 33, 6),
    # more tokens: MFMA tiles (32 tokens up to 4096), ragged in tokens and experts (64-wide tiles)
    (9, 1024, 256, 7), (33, 512, 70, 8), (100, 5120, 256, 9), (1000, 1024, 130, 10), (2048, 5120, 256, 11),
    (40, 128, 1, 12),
    (77, 320, 65, 13),        # 5 K stages: uneven split over the four waves
    # wide routers and a long hidden size
    (4, 8192, 300, 14), (8, 1024, 1024, 15), (130, 2048, 1000, 16), (65, 8192, 256, 17),
    # above 4096 tokens: 64-token tiles
    (5000, 512, 70, 18), (4097, 1024, 256, 19),
]


@pytest.mark.parametrize("T,H,E,seed", CASES)
def test_router_logits_parity(T, H, E, seed):
    got, ref, tol = run(T, H, E, seed)
    assert got.shape == (T, E)
    err = np.abs(got - ref)
    worst = float(np.max(err / tol))
    assert np.all(err <= tol), f"T={T} H={H} E={E}: worst err/bound {worst:.3f}"
    log(f"router T={T} H={H} E={E}: max|err| {err.max():.2e}, worst err/bound {worst:.3f}")


def test_router_logits_deterministic_and_zero_tokens():
    xb, _, wb, _ = wls.router_problem(21, 300, 1024, 256)
    xd, wd = to_dev(xb, torch.int16), to_dev(wb, torch.int16)
    a = B.moe_router_logits(xd, wd)
    b = B.moe_router_logits(xd, wd)
    x1 = B.moe_router_logits(xd[:4].contiguous(), wd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    empty = B.moe_router_logits(torch.empty((0, 1024), dtype=torch.int16, device="cuda:0"), wd)
    assert empty.shape == (0, 256)
    with pytest.raises(B.MoeError) as err:
        B.moe_router_logits(torch.zeros((2, 100), dtype=torch.int16, device="cuda:0"),
                            torch.zeros((8, 100), dtype=torch.int16, device="cuda:0"))
    assert B.STATUS[err.value.status] == "MOE_ERR_SHAPE"
    # the GEMV rows and the MFMA rows agree within the bound of each
    ref = oracle.router_logits(wls.bf16_bits_to_f32(xb[:4]), wls.bf16_bits_to_f32(wb))
    tol = bound(wls.bf16_bits_to_f32(xb[:4]), wls.bf16_bits_to_f32(wb))
    assert np.all(np.abs(a[:4].cpu().numpy() - ref) <= tol)
    assert np.all(np.abs(x1.cpu().numpy() - ref) <= tol)
    log("router: deterministic, T=0 no-op, bad H refused")


@pytest.mark.parametrize("T", [1, 8, 64])
def test_router_then_route_topk(T):
    """The logits feed moe_route_topk; the top-k decision is taken by both
    sides on the same fp32 logits (the device's), so ids are compared
    bit-exactly against the oracle's routing of those logits."""
    H, E, k = 5120, 256, 8
    xb, _, wb, _ = wls.router_problem(30 + T, T, H, E)
    lg = B.moe_router_logits(to_dev(xb, torch.int16), to_dev(wb, torch.int16))
    r = B.moe_route_topk(lg, k)
    torch.cuda.synchronize()
    ids, w = oracle.route_topk(lg.cpu().numpy(), k)
    assert np.array_equal(r.topk_ids.cpu().numpy(), ids)
    assert float(np.max(np.abs(r.topk_w.cpu().numpy() - w))) <= 1e-6
    log(f"router -> route_topk T={T}: ids bit-exact")


@pytest.mark.parametrize("T", [1, 100])
def test_router_and_layer_in_one_graph(T):
    """Router logits, then route + layer (moe_w4a16_route_forward), captured
    in one HIP graph: every replay, with unrelated eager work between them,
    gives the eager result bit for bit (the router needs no workspace and
    allocates nothing)."""
    H, I, E, k = 1024, 512, 32, 4
    _, ms, _, _, _ = wls.random_problem(50 + T, T, H, I, E, k)
    xb, _, wb, _ = wls.router_problem(60 + T, T, H, E)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in ms)
    xd, wd = to_dev(xb, torch.int16), to_dev(wb, torch.int16)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda:0")
    route = B.Routing.empty(T, E, k, "cuda:0")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda:0")
    ws = B.forward_workspace(T, H, I, E, k, "cuda:0")

    def step():
        B.moe_router_logits(xd, wd, out=lg)
        B.moe_w4a16_route_forward(lg, xd, gate, up, down, k, routing=route, out=out, ws=ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lg = out.clone(), lg.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out.fill_(i + 1)
        lg.fill_(float("nan"))
        B.moe_router_logits(wd[:1].contiguous(), wd)             # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lg, ref_lg), f"replay {i}: logits"
        assert torch.equal(out, ref_out), f"replay {i}: output"
    log(f"router + route_forward graph T={T}: 3 replays bit-identical")


# ------------------------------------------------------------------ router + route in one call
ROUTER_ROUTE_CASES = [
    # decode token counts: one launch (every workgroup a ticket, the last one routes)
    (1, 5120, 256, 8), (2, 1024, 64, 4), (8, 5120, 256, 8), (4, 2048, 300, 16), (8, 1024, 1024, 8),
    (1, 128, 7, 7), (3, 512, 33, 32),
    # other shapes: the router kernels, then the route kernels
    (9, 1024, 256, 8), (100, 512, 64, 4),
]


@pytest.mark.parametrize("T,H,E,k", ROUTER_ROUTE_CASES)
def test_router_route_equals_router_then_route(T, H, E, k):
    """moe_router_route_topk gives the logits of moe_router_logits and the
    routing of moe_route_topk on them, bit for bit; the ids also match the
    oracle's routing of those logits; repeated calls on one workspace keep
    working (the ticket word is left at zero); guard bands stay intact."""
    from gpu_util import Guarded, check_guards, guarded_routing
    xb, _, wb, _ = wls.router_problem(700 + T + E, T, H, E)
    xd, wd = to_dev(xb, torch.int16), to_dev(wb, torch.int16)
    lg_ref = B.moe_router_logits(xd, wd)
    r_ref = B.moe_route_topk(lg_ref, k)
    torch.cuda.synchronize()
    ws = Guarded((B.lib().moe_router_route_workspace_size(T, E, k),), torch.uint8)
    ws.t.zero_()
    for rep in range(3):
        r, parts = guarded_routing(T, E, k)
        parts["logits"] = Guarded((T, E), torch.float32)
        B.moe_router_route_topk(xd, wd, k, logits=parts["logits"].t, routing=r, ws=ws.t)
        torch.cuda.synchronize()
        check_guards(parts, f"router_route T{T} E{E} k{k} call {rep}")
        ws.check(f"router_route workspace call {rep}")
        assert int(ws.t[:4].view(torch.int32)[0]) == 0, "ticket word not left at zero"
        assert torch.equal(parts["logits"].t, lg_ref)
        for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
            assert torch.equal(getattr(r, name), getattr(r_ref, name)), (rep, name)
    ids, w = oracle.route_topk(lg_ref.cpu().numpy(), k)
    assert np.array_equal(r.topk_ids.cpu().numpy(), ids)
    assert float(np.max(np.abs(r.topk_w.cpu().numpy() - w))) <= 1e-6
    log(f"router_route T={T} H={H} E={E} k={k}: identical to router + route_topk")


@pytest.mark.parametrize("T", [1, 8])
def test_router_route_and_layer_in_one_graph(T):
    """moe_router_route_topk then moe_w4a16_forward captured in one HIP graph:
    every replay reproduces the eager output and routing bit for bit."""
    H, I, E, k = 1024, 512, 32, 4
    _, ms, _, _, _ = wls.random_problem(80 + T, T, H, I, E, k)
    xb, _, wb, _ = wls.router_problem(90 + T, T, H, E)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in ms)
    xd, wd = to_dev(xb, torch.int16), to_dev(wb, torch.int16)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda:0")
    route = B.Routing.empty(T, E, k, "cuda:0")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda:0")
    ws = B.forward_workspace(T, H, I, E, k, "cuda:0")
    rws = B.router_route_workspace(T, E, k, "cuda:0")

    def step():
        B.moe_router_route_topk(xd, wd, k, logits=lg, routing=route, ws=rws)
        B.moe_w4a16_forward(xd, gate, up, down, route, out=out, ws=ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_ids = out.clone(), route.topk_ids.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out.fill_(i + 1)
        route.topk_ids.fill_(-1)
        B.moe_router_logits(wd[:1].contiguous(), wd)             # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}: output"
        assert torch.equal(route.topk_ids, ref_ids), f"replay {i}: ids"
