"""Oracle pins: the MoE layer in fp64 (CPU)."""
import numpy as np

import pins
from oracle import moe as omoe
from oracle import routing as ort
from nvfp4_weight_only_moe_amd import workloads as wls


def tiny_problem():
    wl = wls.WORKLOADS[0]
    ms = [wls.masters(wl, p) for p in (wls.GATE, wls.UP, wls.DOWN)]
    layer = pins._pack_layer(ms)
    _, x = wls.activations(wl)
    ids, w = ort.route_topk(wls.logits(wl), wl.k)
    return wl, ms, layer, x, ids, w


def test_bruteforce_loops_on_tiny_layer():
    _, _, layer, x, ids, w = tiny_problem()
    pins.pin_bruteforce_layer(x, layer, ids, w)


def test_reduces_to_textbook_swiglu_mlp():
    pins.pin_textbook_mlp()


def test_one_hot_activation_reads_weight_columns():
    pins.pin_one_hot_columns()


def test_magnitude_against_unquantized_layer():
    _, ms, layer, x, ids, w = tiny_problem()
    ratio, rel = pins.pin_magnitude(x, layer, ids, w, ms)
    print(f"norm ratio {ratio:.4f}, relative error vs unquantized {rel:.4f}")


def test_token_subset_matches_full():
    _, _, layer, x, ids, w = tiny_problem()
    full = omoe.moe_forward(x, layer, ids, w)
    part = omoe.moe_forward(x, layer, ids, w, tokens=[3, 0, 11])
    # BLAS may block differently for fewer rows: equal up to fp64 rounding
    assert np.allclose(part[[0, 3, 11]], full[[0, 3, 11]], rtol=1e-13, atol=1e-16)
    assert not part[1].any()


def test_linear_of_representable_weight():
    pins.pin_linear_exact()
    pins.pin_linear_exact(seed=3)


def test_shared_expert_is_textbook_mlp():
    pins.pin_shared_expert_textbook()
