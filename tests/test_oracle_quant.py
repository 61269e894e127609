"""Oracle pins: NVFP4 quantization and dequantization (CPU)."""
import numpy as np
import pytest

import pins
from oracle import nvfp4 as onv


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_roundtrip_of_representable_tensor(seed):
    pins.pin_exact_roundtrip(seed)


def test_nibble_order():
    pins.pin_nibble_order()


@pytest.mark.parametrize("seed", [0, 7])
def test_scale_rule_and_nearest_codes(seed):
    pins.pin_scale_rule(seed)


def test_zero_and_underflowing_tensors():
    pins.pin_zero_and_tiny_tensors()


def test_roundtrip_cosine_band():
    cos = pins.pin_roundtrip_cosine_band()
    print(f"round-trip cosine of N(0, 0.02) weights: {cos:.5f}")


def test_dequant_error_bounded_by_half_step():
    r = np.random.default_rng(3)
    w = (0.02 * r.standard_normal((32, 256))).astype(np.float32)
    packed, scales, g = onv.quantize(w)
    back = onv.dequantize(packed, scales, g)
    s = onv.e4m3_decode(scales)
    d = np.repeat(s * float(g), 16, axis=1)
    # the widest E2M1 gap is 4 -> 6, so no element moves by more than d
    # (plus saturation slack from the E4M3 rounding of the group scale)
    assert np.all(np.abs(back.astype(np.float64) - w) <= d * 1.0 + 1e-12)


def test_quantize_rejects_bad_input():
    with pytest.raises(ValueError):
        onv.quantize(np.zeros((2, 48), np.float32))
    w = np.zeros((2, 32), np.float32)
    w[0, 0] = np.nan
    with pytest.raises(ValueError):
        onv.quantize(w)
