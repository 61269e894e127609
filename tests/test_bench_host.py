"""Host logic of the benchmark: which roofline binds a kernel at a workload.
No GPU: only the arithmetic of the roofline choice is exercised."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


H, I = 5120, 1536


def test_packed_bytes_of_an_expert(bench):
    # codes (N*K/2) + one E4M3 scale per 16 codes (N*K/16) + the FP32 global scale
    assert bench.packed_bytes(I, H) == I * H // 2 + I * H // 16 + 4
    assert 2 * bench.packed_bytes(I, H) == 8_847_368


@pytest.mark.parametrize("rows_per_expert,bound", [(32, "hbm"), (80, "hbm"), (100, "mfma"), (640, "mfma")])
def test_grouped_gemm_bound_follows_rows_per_expert(bench, rows_per_expert, bound):
    """Gate/up GEMM over 256 touched experts: weights 8,847,368 B each at
    8 TB/s against 4*H*I flop per row at 2.5 PFLOP/s cross near 88 rows."""
    experts = 256
    rows = experts * rows_per_expert
    w = experts * 2 * bench.packed_bytes(I, H) + rows * H * 2
    f = 4.0 * rows * H * I
    r = bench.make_roofline("gemm_gateup", 1000.0, w, f, None)
    assert r["bound"] == bound
    assert r["other"]["bound"] != bound
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)


def test_decode_kernel_is_hbm_bound_without_flops(bench):
    r = bench.make_roofline("dec_gateup_route", 17.75, 70_790_208, None, 70_000_000)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and "other" not in r
    assert r["achieved"] == pytest.approx(70_790_208 / 17.75e-6 / 1e9, rel=1e-4)
    assert r["traffic"] == 70_000_000
