"""GPU parity of the single-expert entry points against the oracle: the dense
NVFP4 projection (moe_w4a16_linear) and the shared expert
(moe_w4a16_shared_expert).  Inputs are the seeded generators' (workloads);
expected values come from the oracle alone, which quantizes the same masters
itself."""
import numpy as np
import pytest
import torch

import oracle
from oracle import moe as omoe
from nvfp4_weight_only_moe_amd import binding as B
from nvfp4_weight_only_moe_amd import workloads as wls
from gpu_util import bf16_bits_to_f64, compare_out, log, oracle_layer_from_masters, pack_gpu, to_dev

pytestmark = pytest.mark.gpu

LINEAR_CASES = [
    # 1-8 tokens, K % 1024 == 0: the decode gate/up kernel with one weight stack
    (1, 1024, 512, 11), (2, 2048, 1536, 12), (8, 5120, 1536, 13), (1, 5120, 5120, 14),
    (3, 1024, 100, 15),                      # N not a multiple of the 8- or 16-row blocks
    # the grouped down GEMM with one expert, then the combine
    (9, 1024, 512, 16), (100, 1536, 1024, 17), (5, 384, 256, 19),
    (300, 1024, 512, 18),                    # >= 256 rows: the LDS-pipelined kernel
]


@pytest.mark.parametrize("T,K,N,seed", LINEAR_CASES)
def test_linear_parity(T, K, N, seed):
    _, ms, xb, x, _ = wls.random_problem(seed, T, K, N, 1, 1)
    w = ms[0]                                                    # [1, N, K]
    out = B.moe_w4a16_linear(to_dev(xb, torch.int16), pack_gpu(w))
    torch.cuda.synchronize()
    codes, scales, g = oracle.quantize_layer(w)
    ref = omoe.linear(x, codes[0], scales[0], g[0])
    compare_out(bf16_bits_to_f64(out), ref, f"linear T={T} K={K} N={N}")


def test_linear_zero_tokens_and_bad_shape():
    _, ms, xb, _, _ = wls.random_problem(31, 2, 1536, 100, 1, 1)
    wt = pack_gpu(ms[0])
    empty = B.moe_w4a16_linear(torch.empty((0, 1536), dtype=torch.int16, device="cuda:0"), wt)
    assert empty.shape == (0, 100)
    # 2 tokens with K % 1024 != 0 take the grouped GEMM, which needs N % 256 == 0
    with pytest.raises(B.MoeError) as err:
        B.moe_w4a16_linear(to_dev(xb, torch.int16), wt)
    assert B.STATUS[err.value.status] == "MOE_ERR_SHAPE"
    log("linear: T=0 no-op, unsupported shape refused")


SHARED_CASES = [
    (1, 1024, 512, 21), (4, 1024, 512, 22), (8, 2048, 1024, 23),    # decode kernels
    (40, 1024, 512, 24), (300, 1024, 512, 25),                       # grouped / pipelined GEMMs
    (1, 5120, 1536, 26), (8, 5120, 1536, 27),                        # the model's shapes
    # one-expert decode mode across its templates: H / 1024 = 3, 4, 8 and
    # I / 512 = 2, 3, 4 with 2-, 4- and 8-token blocks
    (2, 3072, 2048, 28), (3, 4096, 1024, 29), (5, 8192, 1536, 30),
]


@pytest.mark.parametrize("T,H,I,seed", SHARED_CASES)
def test_shared_expert_parity(T, H, I, seed):
    _, ms, xb, x, _ = wls.random_problem(seed, T, H, I, 1, 1)
    gate, up, down = (pack_gpu(m) for m in ms)
    out = B.moe_w4a16_shared_expert(to_dev(xb, torch.int16), gate, up, down)
    torch.cuda.synchronize()
    ref = omoe.shared_expert_forward(x, oracle_layer_from_masters(ms))
    compare_out(bf16_bits_to_f64(out), ref, f"shared expert T={T} H={H} I={I}")


@pytest.mark.parametrize("T,H,I", [(6, 1024, 512), (1, 5120, 1536), (8, 2048, 2048), (20, 1024, 512)])
def test_shared_expert_matches_one_expert_forward(T, H, I):
    """The entry point is the routed forward with one expert, k = 1, weight 1:
    the same arithmetic, the same bits (1-8 tokens: the decode kernels in
    their one-expert mode against the routed decode kernels)."""
    _, ms, xb, _, _ = wls.random_problem(41, T, H, I, 1, 1)
    gate, up, down = (pack_gpu(m) for m in ms)
    xd = to_dev(xb, torch.int16)
    shared = B.moe_w4a16_shared_expert(xd, gate, up, down)
    r = B.moe_route_topk(torch.zeros((T, 1), dtype=torch.float32, device="cuda:0"), 1)
    routed = B.moe_w4a16_forward(xd, gate, up, down, r)
    torch.cuda.synchronize()
    assert torch.equal(shared, routed)
    log(f"shared expert T={T} H={H} I={I}: bit-identical to the one-expert routed forward")
