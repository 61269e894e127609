"""The no-allocation entry point (moe_w4a16_route_forward_noalloc) against
the entry point it varies (moe_w4a16_route_forward): two calls in a row on
the library's own device array, the second with a smaller input, each equal
to the existing entry point's output bit for bit (and so within the
forward's bar); a shape whose workspace exceeds the array is refused."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, Problem, bf16_bits_to_f64, compare_out, log, to_dev
from nvfp4_weight_only_moe_amd import binding as B

pytestmark = pytest.mark.gpu


def _both(p):
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    lg, xb = to_dev(p.logits), to_dev(p.xb, torch.int16)
    ref, r_ref = B.moe_w4a16_route_forward(lg, xb, gate, up, down, p.k)
    out = torch.full_like(ref, 0x7FBF)
    got, r = B.moe_w4a16_route_forward_noalloc(lg, xb, gate, up, down, p.k, out=out)
    torch.cuda.synchronize()
    return ref, r_ref, got, r


def test_noalloc_matches_route_forward_twice_then_smaller():
    cases = [(300, 1024, 512, 16, 4, 900),     # grouped GEMMs, route scratch in the array
             (8, 2048, 1024, 32, 8, 901),      # smaller: decode kernels
             (1, 1024, 512, 8, 2, 902)]        # smaller still: one token, route inside gate/up
    for T, H, I, E, k, seed in cases:
        p = Problem(T, H, I, E, k, seed)
        need = B.moe_w4a16_workspace_size(T, H, I, E, k)
        ref, r_ref, got, r = _both(p)
        for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_slots", "slot_pos"):
            assert torch.equal(getattr(r, name), getattr(r_ref, name)), (T, name)
        assert torch.equal(got, ref), T
        compare_out(bf16_bits_to_f64(got), bf16_bits_to_f64(ref), f"noalloc T{T} (workspace {need} B)")
        log(f"noalloc T{T}: identical to moe_w4a16_route_forward")


def test_noalloc_refuses_a_workspace_beyond_the_array():
    T, H, I, E, k = 4096, 1024, 512, 16, 4      # h and y rows of 16,384 token-expert pairs: 48 MiB
    need = B.moe_w4a16_workspace_size(T, H, I, E, k)
    assert need > (32 << 20)
    p = Problem(T, H, I, E, k, 903)
    gate, up, down = (B.moe_w4a16_quantize_pack(to_dev(m)) for m in p.ms)
    out = torch.full((T, H), 7, dtype=torch.int16, device=DEV)
    with pytest.raises(B.MoeError) as err:
        B.moe_w4a16_route_forward_noalloc(to_dev(p.logits), to_dev(p.xb, torch.int16), gate, up, down, k, out=out)
    assert B.STATUS[err.value.status] == "MOE_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert bool((out == 7).all())
