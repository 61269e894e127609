"""Pins of the router oracle (oracle/router.py) to values fixed by the
definition of the linear gate, not by the oracle's own formula."""
import numpy as np
import pytest

import oracle
from nvfp4_weight_only_moe_amd import workloads as wls


def test_one_hot_rows_pick_single_weights():
    """Row t = unit vector j_t gives logits[t, e] = W[e, j_t] exactly, for
    every expert: a transposed operand or a swapped output axis fails (T, E
    and H all differ)."""
    T, H, E = 5, 48, 7
    _, _, _, w = wls.router_problem(3, T, H, E)
    js = [0, 47, 13, 13, 30]
    x = np.zeros((T, H))
    for t, j in enumerate(js):
        x[t, j] = 1.0
    lg = oracle.router_logits(x, w)
    assert lg.shape == (T, E)
    for t, j in enumerate(js):
        for e in range(E):
            assert lg[t, e] == float(w[e, j])


def test_constant_rows_closed_form():
    """x[t, :] = c_t and W[e, :] = d_e give H * c_t * d_e, exact in fp64 for
    these small dyadic values."""
    T, H, E = 3, 64, 4
    c = np.array([1.0, -0.5, 2.0])
    d = np.array([0.25, -1.0, 3.0, 0.0])
    x = np.repeat(c[:, None], H, axis=1)
    w = np.repeat(d[:, None], H, axis=1)
    lg = oracle.router_logits(x, w)
    for t in range(T):
        for e in range(E):
            assert lg[t, e] == H * c[t] * d[e]


def test_alternating_signs_cancel_and_negation_flips():
    """A row of alternating +1/-1 against a constant weight row sums to 0;
    negating the weights negates every logit exactly."""
    T, H, E = 4, 32, 6
    _, x, _, w = wls.router_problem(5, T, H, E)
    alt = np.array([1.0 if i % 2 == 0 else -1.0 for i in range(H)])
    flat = np.full((1, H), 0.75)
    assert oracle.router_logits(alt[None, :], flat)[0, 0] == 0.0
    np.testing.assert_array_equal(oracle.router_logits(x, -w), -oracle.router_logits(x, w))


def test_logit_scale_of_the_generator():
    """The generator's weights N(0, 1/H) give logits of about unit variance
    (the drawn logits of the workloads are N(0, 1))."""
    _, x, _, w = wls.router_problem(7, 64, 1024, 256)
    lg = oracle.router_logits(x, w)
    assert 0.8 < lg.std() < 1.2


def test_shape_mismatch_refused():
    with pytest.raises(ValueError):
        oracle.router_logits(np.zeros((2, 8)), np.zeros((3, 9)))


# Planted mistakes in the router oracle must each trip one of the pins above.
_MUTANTS = {
    # the expert axis reversed (a wrong row index into W)
    "experts reversed": lambda x, w: np.asarray(x, np.float64) @ np.asarray(w, np.float64)[::-1].T,
    "dropped last column": lambda x, w: np.asarray(x, np.float64)[:, :-1] @ np.asarray(w, np.float64)[:, :-1].T,
    "bias of one": lambda x, w: np.asarray(x, np.float64) @ np.asarray(w, np.float64).T + 1.0,
    "sign flipped": lambda x, w: -(np.asarray(x, np.float64) @ np.asarray(w, np.float64).T),
    "mean instead of sum": lambda x, w: (np.asarray(x, np.float64) @ np.asarray(w, np.float64).T) / np.asarray(x).shape[1],
}


def _router_pins():
    test_one_hot_rows_pick_single_weights()
    test_constant_rows_closed_form()
    test_alternating_signs_cancel_and_negation_flips()
    test_logit_scale_of_the_generator()


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_planted_router_mistake_is_caught(name, monkeypatch):
    import oracle.router as orouter
    mutant = _MUTANTS[name]
    monkeypatch.setattr(orouter, "router_logits", mutant)
    monkeypatch.setattr(oracle, "router_logits", mutant)
    with pytest.raises(AssertionError):
        _router_pins()
