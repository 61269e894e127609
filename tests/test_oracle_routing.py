"""Oracle pins: top-k routing and the expert-sorted permutation (CPU)."""
import numpy as np
import pytest

import pins
from oracle import routing as ort
from nvfp4_weight_only_moe_amd import workloads as wls


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_route_bruteforce_workloads(cfg):
    wl = wls.WORKLOADS[cfg]
    lg = wls.logits(wl)
    pins.pin_route_bruteforce(lg, wl.k)
    ids, _ = ort.route_topk(lg, wl.k)
    pins.pin_permutation(ids, wl.E)


def test_route_ties_take_lower_index():
    lg = np.zeros((3, 8), np.float32)
    lg[1, [2, 5, 6]] = 1.0
    lg[2] = [3, 3, -1, 3, 0.5, 0.5, -0.0, 0.0]
    pins.pin_route_bruteforce(lg, 3)
    ids, w = ort.route_topk(lg, 3)
    assert list(ids[0]) == [0, 1, 2]
    assert list(ids[1]) == [2, 5, 6]
    assert list(ids[2]) == [0, 1, 3]
    assert np.allclose(w[0], 1 / 3)


def test_route_k_equals_e_and_k_one():
    r = np.random.default_rng(0)
    lg = r.standard_normal((9, 16)).astype(np.float32)
    pins.pin_route_bruteforce(lg, 16)
    pins.pin_route_bruteforce(lg, 1)
    ids, w = ort.route_topk(lg, 1)
    assert np.all(w == 1.0)


def test_permutation_random_and_skewed():
    r = np.random.default_rng(1)
    pins.pin_permutation(r.integers(0, 32, size=(50, 4)), 32)
    pins.pin_permutation(np.zeros((7, 3), np.int64) + 5, 8)       # one hot expert
    pins.pin_permutation(np.zeros((0, 2), np.int64), 4)            # empty


def test_zipf_workload_is_skewed():
    wl = wls.WORKLOADS[4]
    lg = wls.logits(wl, T=2048)
    ids, _ = ort.route_topk(lg, wl.k)
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    # the hottest expert takes far more than the uniform share (64 at T=2048)
    assert counts.max() > 10 * 64
    assert (counts == 0).sum() > 10
