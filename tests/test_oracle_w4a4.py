"""Oracle pins: the W4A4 NVFP4 variant (activations quantized too), CPU."""
import pytest

import pins


@pytest.mark.parametrize("seed", [0, 1])
def test_activation_exact_roundtrip(seed):
    pins.pin_act_exact_roundtrip(seed)


@pytest.mark.parametrize("seed", [0, 5])
def test_activation_scale_rule_and_bruteforce(seed):
    pins.pin_act_scale_rule(seed)


def test_bad_input_scales_are_refused():
    pins.pin_input_scale_refusal()


def test_placeholder_scale_underflows_to_zero():
    pins.pin_placeholder_underflow()


def test_representable_activations_match_w4a16():
    pins.pin_w4a4_representable_x()


def test_bruteforce_layer():
    pins.pin_w4a4_bruteforce()


def test_magnitude_bands():
    ratio, d = pins.pin_w4a4_magnitude()
    print(f"W4A4 norm ratio to the unquantized layer {ratio:.4f}; relative difference to W4A16 {d:.4f}")
