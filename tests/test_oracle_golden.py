"""The oracle still gives the answers stored in tests/golden (CPU).

The stored file was written by tests/golden/make_golden.py, which calls only
the oracle; see that script for why it exists."""
import json
import os

import numpy as np

from tests_golden_loader import load_golden_builder


def test_oracle_matches_stored_tiny_layer():
    here = os.path.join(os.path.dirname(__file__), "golden")
    with open(os.path.join(here, "tiny_layer_oracle.json")) as f:
        stored = json.load(f)
    now = load_golden_builder().build()
    assert now["projections"] == stored["projections"]
    assert now["route"] == stored["route"]
    for a, b in zip(now["out_rows_0_and_15_first8_hex"], stored["out_rows_0_and_15_first8_hex"]):
        assert np.allclose([float.fromhex(v) for v in a], [float.fromhex(v) for v in b],
                           rtol=1e-12, atol=0)
    assert abs(now["out_frobenius"] - stored["out_frobenius"]) <= 1e-12 * stored["out_frobenius"]
