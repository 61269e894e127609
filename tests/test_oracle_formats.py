"""Oracle pins: the E2M1 and E4M3 formats (CPU)."""
import pins


def test_e2m1_table():
    pins.pin_e2m1_table()


def test_e4m3_decode_matches_torch():
    pins.pin_e4m3_decode_vs_torch()


def test_e4m3_encode_midpoints_and_saturation():
    pins.pin_e4m3_encode_midpoints()


def test_e4m3_encode_matches_torch_below_464():
    pins.pin_e4m3_encode_vs_torch()


def test_e2m1_encode_midpoints_signs_saturation():
    pins.pin_e2m1_encode_midpoints()
