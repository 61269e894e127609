"""GPU parity: top-k ids, counts, offsets and the permutation are bit-exact
against the oracle; routing weights within 1e-6.  Through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import log, to_dev
from nvfp4_weight_only_moe_amd import binding as B
from nvfp4_weight_only_moe_amd import workloads as wls

pytestmark = pytest.mark.gpu


def check_route(logits, k, where):
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    r = B.moe_route_topk(to_dev(logits), k)
    torch.cuda.synchronize()
    ids, w = oracle.route_topk(logits, k)
    counts, offsets, sorted_slots, slot_pos = oracle.permutation(ids, E)
    assert np.array_equal(r.topk_ids.cpu().numpy(), ids), f"{where}: ids"
    dw = float(np.max(np.abs(r.topk_w.cpu().numpy().astype(np.float64) - w))) if T else 0.0
    assert dw <= 1e-6, (where, dw)
    assert np.array_equal(r.counts.cpu().numpy(), counts), f"{where}: counts"
    assert np.array_equal(r.offsets.cpu().numpy(), offsets), f"{where}: offsets"
    assert np.array_equal(r.sorted_slots.cpu().numpy(), sorted_slots), f"{where}: sorted_slots"
    assert np.array_equal(r.slot_pos.cpu().numpy(), slot_pos), f"{where}: slot_pos"
    log(f"route {where}: T={T} E={E} k={k} bit-exact, max|dw|={dw:.2e}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_route_workloads(cfg):
    wl = wls.WORKLOADS[cfg]
    check_route(wls.logits(wl), wl.k, wl.name)


@pytest.mark.parametrize("T,E,k", [(1, 8, 1), (7, 64, 4), (64, 256, 8), (65, 256, 8), (300, 100, 3),
                                   (129, 1024, 32), (50, 32, 32), (1000, 16, 2),
                                   # the decode-sized route (T <= 16, T * k <= 64) at its limits and
                                   # for every logits-per-lane variant, and just past them
                                   (16, 1024, 4), (2, 128, 32), (16, 100, 1), (3, 513, 5), (1, 1024, 8),
                                   (17, 64, 2), (9, 256, 8)])
def test_route_shapes(T, E, k):
    r = np.random.default_rng(T * 1000 + E)
    check_route(r.standard_normal((T, E)).astype(np.float32), k, f"random-{T}-{E}-{k}")


@pytest.mark.parametrize("E", [64, 256, 300])
@pytest.mark.parametrize("T", [5, 200])
def test_route_ties_and_skew(T, E):
    """Exact ties (several logits per lane of the selecting wave when E > 64),
    signed zeros and a dominant expert."""
    r = np.random.default_rng(T * 7 + E)
    lg = r.integers(-2, 3, size=(T, E)).astype(np.float32)     # many exact ties
    lg[:, 0] = -0.0
    lg[:, 1] = 0.0
    check_route(lg, 8, f"ties-{T}")
    sk = r.standard_normal((T, E)).astype(np.float32)
    sk[:, 5] += 50.0                                             # every token picks expert 5
    check_route(sk, 2, f"skew-{T}")


def test_route_empty():
    r = B.moe_route_topk(torch.zeros((0, 16), dtype=torch.float32, device="cuda"), 2)
    torch.cuda.synchronize()
    assert r.topk_ids.numel() == 0


def test_route_deterministic():
    wl = wls.WORKLOADS[4]
    lg = to_dev(wls.logits(wl))
    a = B.moe_route_topk(lg, wl.k)
    b = B.moe_route_topk(lg, wl.k)
    torch.cuda.synchronize()
    for f in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
