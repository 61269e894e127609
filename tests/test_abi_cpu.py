"""The C ABI on the CPU: the library loads, exports what the header declares,
and refuses bad arguments on the host before touching the device.

Every call here fails (or is a T = 0 no-op) before any HIP call, so nothing
needs a GPU.  Device pointers are fake, 16-byte aligned integers.
"""
import ctypes

import pytest

from nvfp4_weight_only_moe_amd import binding as b

A = 0x10000  # a fake, aligned device address


def T_(E, N, K, base=A):
    return b.NVFP4TensorC(E, N, K, base, base + 0x100000, base + 0x200000)


@pytest.fixture(scope="module")
def L():
    return b.lib()


def test_library_exports_every_declared_symbol(L):
    names = b.header_symbols()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in b.STATUS.items():
        assert b.status_string(code).startswith(name)
    assert "UNKNOWN" in b.status_string(-99)


def fwd(L, x=A, T=4, H=256, I=128, E=8, k=2, gate=None, up=None, down=None, ptr=A, out=A + 0x800000,
        ws=A + 0x900000, ws_bytes=1 << 30):
    gate = gate or T_(E, I, H)
    up = up or T_(E, I, H, A + 0x1000000)
    down = down or T_(E, H, I, A + 0x2000000)
    p = [ptr] * 6
    return L.moe_w4a16_forward(x, T, H, I, E, k, ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down),
                               *p, out, ws, ws_bytes, None)


def test_forward_argument_errors(L):
    assert fwd(L, T=0) == b.MOE_OK                                 # no-op
    assert fwd(L, T=-1) == -2                                      # SHAPE
    assert fwd(L, H=200) == -2                                     # H % 256
    assert fwd(L, I=100) == -2                                     # I % 128
    assert fwd(L, k=9) == -4                                       # k > E
    assert fwd(L, E=2000, k=2) == -4                               # E > 1024
    assert fwd(L, k=33, E=64) == -4                                # k > 32
    assert fwd(L, x=0) == -1                                       # null x
    assert fwd(L, ptr=0) == -1                                     # null routing arrays
    assert fwd(L, x=A + 4) == -3                                   # misaligned
    assert fwd(L, out=A) == -1                                     # out aliases x
    assert fwd(L, ws=0) == -7                                      # no workspace
    assert fwd(L, ws_bytes=16) == -7                               # workspace too small
    assert fwd(L, gate=T_(8, 128, 512)) == -2                      # wrong gate K
    assert fwd(L, down=T_(8, 128, 256)) == -2                      # down not [H, I]
    assert fwd(L, up=b.NVFP4TensorC(8, 128, 256, A, A, 0)) == -1   # missing global scale
    assert fwd(L, up=b.NVFP4TensorC(8, 128, 256, A + 8, A, A)) == -3
    assert L.moe_w4a16_forward(A, 4, 256, 128, 8, 2, None, None, None, A, A, A, A, A, A, A, A, 1 << 30, None) == -1


def test_route_argument_errors(L):
    def r(T=4, E=8, k=2, ptr=A, ws=A, ws_bytes=1 << 20):
        return L.moe_route_topk(ptr, T, E, k, ptr, ptr, ptr, ptr, ptr, ptr, ws, ws_bytes, None)
    assert r(T=0) == b.MOE_OK
    assert r(T=-1) == -2
    assert r(k=0) == -2
    assert r(k=9) == -4
    assert r(E=1025, k=2) == -4
    assert r(ptr=0) == -1
    assert r(ptr=A + 2) == -3
    big = 100000
    assert L.moe_route_workspace_size(big, 256, 8) > 0
    assert r(T=big, E=256, k=8, ws_bytes=0) == -7
    assert r(T=big, E=256, k=8, ws=0) == -7
    assert L.moe_route_workspace_size(1, 256, 8) == 0


def test_quantize_dequantize_validate_argument_errors(L):
    t = T_(2, 64, 256)
    assert L.moe_w4a16_quantize_pack(None, 2, 64, 256, ctypes.byref(t), None) == -1
    assert L.moe_w4a16_quantize_pack(A + 0x4000000, 2, 64, 48, ctypes.byref(t), None) == -2   # K % 32
    assert L.moe_w4a16_quantize_pack(A + 0x4000000, 2, 64, 128, ctypes.byref(t), None) == -2  # K mismatch
    assert L.moe_w4a16_quantize_pack(A + 0x4000004, 2, 64, 256, ctypes.byref(t), None) == -3
    assert L.moe_w4a16_quantize_pack(A, 2, 64, 256, ctypes.byref(t), None) == -1              # w overlaps out
    assert L.moe_w4a16_quantize_pack(A + 0x4000000, 2, 64, 256, None, None) == -1
    assert L.moe_w4a16_quantize_pack(A + 0x4000000, 2000, 64, 256, ctypes.byref(T_(2000, 64, 256)), None) == -4
    assert L.moe_w4a16_dequantize(ctypes.byref(t), None, None) == -1
    assert L.moe_w4a16_dequantize(ctypes.byref(T_(2, 64, 40)), A, None) == -2
    assert L.moe_w4a16_validate(None, A + 0x4000000, None) == -1
    assert L.moe_w4a16_validate(ctypes.byref(T_(0, 64, 256)), A + 0x4000000, None) == -2
    # the flag word is the caller's: required, aligned, and apart from the tensor
    assert L.moe_w4a16_validate(ctypes.byref(t), None, None) == -7
    assert L.moe_w4a16_validate(ctypes.byref(t), A + 0x4000004, None) == -3
    assert L.moe_w4a16_validate(ctypes.byref(t), A + 0x100000, None) == -1    # the first scale byte


def test_workspace_sizes(L):
    assert L.moe_w4a16_workspace_size(0, 5120, 1536, 256, 8) == 0
    need = L.moe_w4a16_workspace_size(16, 256, 128, 8, 2)
    assert need >= 16 * 2 * (128 * 2 + 256 * 2)
    assert need % 256 == 0


def rfwd(L, logits=A + 0x700000, x=A, T=4, H=256, I=128, E=8, k=2, ptr=A + 0x600000, out=A + 0x800000,
         ws=A + 0x900000, ws_bytes=1 << 30):
    gate, up, down = T_(E, I, H), T_(E, I, H, A + 0x1000000), T_(E, H, I, A + 0x2000000)
    p = [ptr] * 6
    return L.moe_w4a16_route_forward(logits, x, T, H, I, E, k, ctypes.byref(gate), ctypes.byref(up),
                                     ctypes.byref(down), *p, out, ws, ws_bytes, None)


def test_route_forward_argument_errors(L):
    assert rfwd(L, T=0) == b.MOE_OK
    assert rfwd(L, T=-1) == -2
    assert rfwd(L, logits=0) == -1                                  # null logits
    assert rfwd(L, logits=A + 4) == -3
    assert rfwd(L, ptr=0) == -1                                     # null routing outputs
    assert rfwd(L, k=9) == -4
    assert rfwd(L, H=200) == -2
    assert rfwd(L, out=A) == -1                                     # out aliases x
    assert rfwd(L, ws=0) == -7
    assert rfwd(L, ws_bytes=16) == -7


def test_forward_workspace_layout_size(L):
    # h (bf16 [T*k][I]) then y (bf16 [T*k][H]); nothing before them
    T, H, I, E, k = 3, 1024, 512, 16, 4
    assert L.moe_w4a16_workspace_size(T, H, I, E, k) == T * k * I * 2 + T * k * H * 2
    # large T also carries the route scratch
    assert L.moe_w4a16_workspace_size(1000, H, I, E, k) >= (
        1000 * k * (I * 2 + H * 2) + L.moe_route_workspace_size(1000, E, k))


def test_removed_entry_points_are_gone(L):
    # the single-launch decode variant and its hooks were retired
    for name in ("moe_w4a16_workspace_init", "moe_debug_set_decode_variant", "moe_debug_set_decode_wait_limit"):
        assert not hasattr(L, name), name


def test_prefill_variant_hook(L):
    assert L.moe_debug_set_prefill_variant(3) == -1
    assert L.moe_debug_set_prefill_variant(-1) == -1
    assert L.moe_debug_set_prefill_variant(0) == 0
    assert L.moe_debug_set_prefill_variant(1) == 0
    assert L.moe_debug_set_prefill_variant(2) == 0


def lin(L, x=A, T=4, K=1024, N=512, w=None, out=A + 0x800000, ws=A + 0x900000, ws_bytes=1 << 30):
    w = w or T_(1, N, K, A + 0x1000000)
    return L.moe_w4a16_linear(x, T, K, N, ctypes.byref(w), out, ws, ws_bytes, None)


def test_linear_argument_errors(L):
    assert lin(L, T=0) == b.MOE_OK                                 # no-op, any path
    assert lin(L, T=0, N=100, K=1536) == b.MOE_OK
    assert lin(L, T=-1) == -2                                      # SHAPE
    assert lin(L, K=0) == -2
    assert lin(L, w=T_(2, 512, 1024)) == -2                        # a stack of 2: not E = 1
    assert lin(L, w=T_(1, 256, 1024)) == -2                        # N does not match the tensor
    assert lin(L, T=2, K=1536, N=100) == -2                        # GEMM path needs N % 256
    assert lin(L, T=9, K=1000, N=512,
               w=T_(1, 512, 1000)) != b.MOE_OK                     # K not a multiple of 32 (tensor)
    assert lin(L, x=0) == -1                                       # null x
    assert lin(L, x=A + 4) == -3                                   # misaligned
    assert lin(L, out=A) == -1                                     # out overlaps x
    assert lin(L, ws=0) == -7                                      # no workspace
    assert lin(L, ws_bytes=16) == -7                               # workspace too small
    assert L.moe_w4a16_linear_workspace_size(4, 1024, 512) >= 4 * 512 * 2
    assert L.moe_w4a16_linear_workspace_size(0, 1024, 512) == 0


def shx(L, x=A, T=4, H=256, I=128, out=A + 0x800000, ws=A + 0x900000, ws_bytes=1 << 30, gate=None):
    gate = gate or T_(1, I, H)
    up = T_(1, I, H, A + 0x1000000)
    down = T_(1, H, I, A + 0x2000000)
    return L.moe_w4a16_shared_expert(x, T, H, I, ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down),
                                     out, ws, ws_bytes, None)


def test_shared_expert_argument_errors(L):
    assert shx(L, T=0) == b.MOE_OK
    assert shx(L, T=-1) == -2
    assert shx(L, H=200) == -2                                     # H % 256
    assert shx(L, gate=T_(2, 128, 256)) == -2                      # not one expert
    assert shx(L, x=0) == -1
    assert shx(L, out=A) == -1                                     # out aliases x
    assert shx(L, ws=0) == -7
    assert shx(L, ws_bytes=1024) == -7
    need = L.moe_w4a16_shared_expert_workspace_size(4, 256, 128)
    assert need > L.moe_w4a16_workspace_size(4, 256, 128, 1, 1)  # identity routing in front


def rtr(L, x=A, T=4, H=1024, wr=A + 0x100000, E=256, out=A + 0x800000):
    return L.moe_router_logits(x, T, H, wr, E, out, None)


def test_router_logits_argument_errors(L):
    assert rtr(L, T=0) == b.MOE_OK                                 # no-op
    assert rtr(L, T=-1) == -2                                      # SHAPE
    assert rtr(L, H=100) == -2                                     # H % 64 != 0
    assert rtr(L, H=0) == -2
    assert rtr(L, E=0) == -2
    assert rtr(L, x=0) == -1                                       # null pointers
    assert rtr(L, wr=0) == -1
    assert rtr(L, out=0) == -1
    assert rtr(L, x=A + 2) == -3                                   # misaligned
    assert rtr(L, out=A + 0x800004) == -3
    assert rtr(L, out=A + 0x100) == -1                             # logits overlap x
    assert rtr(L, out=A + 0x100000) == -1                          # logits overlap the router weight


def w4(L, x=A, T=4, H=256, I=128, E=8, k=2, sx=0.01, sh=0.02, ptr=A, out=A + 0x800000, ws=A + 0x900000,
       ws_bytes=1 << 30):
    gate, up, down = T_(E, I, H), T_(E, I, H, A + 0x1000000), T_(E, H, I, A + 0x2000000)
    p = [ptr] * 6
    return L.moe_w4a4_forward(x, T, H, I, E, k, ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down),
                              ctypes.c_float(sx), ctypes.c_float(sh), *p, out, ws, ws_bytes, None)


def test_w4a4_argument_errors(L):
    L.moe_w4a4_forward.argtypes = b._SIGS["moe_w4a4_forward"][1]
    assert w4(L, T=0) == b.MOE_OK
    for bad in (0.0, -0.0, -1.0):
        assert w4(L, sx=bad) == -6                                   # BAD_SCALE
        assert w4(L, sh=bad) == -6
        assert w4(L, T=0, sx=bad) == -6                              # refused even as a no-op
    for bad in (float("nan"), float("inf"), float("-inf")):
        assert w4(L, sx=bad) == -5                                   # NONFINITE
        assert w4(L, sh=bad) == -5
    assert w4(L, H=200) == -2
    assert w4(L, x=0) == -1
    assert w4(L, out=A) == -1
    assert w4(L, ws=0) == -7
    need = L.moe_w4a4_workspace_size(4, 256, 128, 8, 2)
    assert need > L.moe_w4a16_workspace_size(4, 256, 128, 8, 2)
    assert w4(L, ws_bytes=need - 1) == -7


def w4r(L, logits=A + 0x3000000, x=A, T=4, H=256, I=128, E=8, k=2, sx=0.01, sh=0.02, ptr=A + 0x3100000,
        out=A + 0x800000, ws=A + 0x900000, ws_bytes=1 << 30):
    gate, up, down = T_(E, I, H), T_(E, I, H, A + 0x1000000), T_(E, H, I, A + 0x2000000)
    p = [ptr] * 6
    return L.moe_w4a4_route_forward(logits, x, T, H, I, E, k, ctypes.byref(gate), ctypes.byref(up),
                                    ctypes.byref(down), ctypes.c_float(sx), ctypes.c_float(sh), *p, out, ws,
                                    ws_bytes, None)


def test_w4a4_route_forward_argument_errors(L):
    L.moe_w4a4_route_forward.argtypes = b._SIGS["moe_w4a4_route_forward"][1]
    assert w4r(L, T=0) == b.MOE_OK
    for bad in (0.0, -1.0):
        assert w4r(L, sx=bad) == -6
        assert w4r(L, sh=bad) == -6
        assert w4r(L, T=0, sh=bad) == -6
    assert w4r(L, sx=float("nan")) == -5
    assert w4r(L, logits=0) == -1
    assert w4r(L, x=0) == -1
    assert w4r(L, H=200) == -2
    assert w4r(L, ws=0) == -7
    assert w4r(L, ws_bytes=L.moe_w4a4_workspace_size(4, 256, 128, 8, 2) - 1) == -7


def test_quantize_activations_argument_errors(L):
    q = L.moe_nvfp4_quantize_activations
    f = ctypes.c_float
    assert q(A, 0, 64, f(1.0), A + 0x100000, A + 0x200000, None) == b.MOE_OK
    assert q(A, 4, 64, f(0.0), A + 0x100000, A + 0x200000, None) == -6
    assert q(A, 4, 64, f(float("nan")), A + 0x100000, A + 0x200000, None) == -5
    assert q(A, 4, 48, f(1.0), A + 0x100000, A + 0x200000, None) == -2       # K % 32
    assert q(A, -1, 64, f(1.0), A + 0x100000, A + 0x200000, None) == -2
    assert q(0, 4, 64, f(1.0), A + 0x100000, A + 0x200000, None) == -1
    assert q(A, 4, 64, f(1.0), A + 4, A + 0x200000, None) == -3
    assert q(A, 4, 64, f(1.0), A + 0x40, A + 0x200000, None) == -1          # codes overlap x


def test_router_route_argument_errors(L):
    def rr(x=A, T=4, H=1024, wr=A + 0x100000, E=256, k=8, lg=A + 0x800000, ptr=A + 0x900000, ws=A + 0xA00000,
           ws_bytes=1 << 20):
        return L.moe_router_route_topk(x, T, H, wr, E, k, lg, ptr, ptr, ptr, ptr, ptr, ptr, ws, ws_bytes, None)
    assert rr(T=0) == b.MOE_OK
    assert rr(T=-1) == -2
    assert rr(H=100) == -2
    assert rr(k=9, E=8) == -4
    assert rr(k=33) == -4
    assert rr(x=0) == -1
    assert rr(lg=A + 0x800004) == -3
    assert rr(ws=0) == -7
    assert rr(ws_bytes=8) == -7
    assert rr(lg=A + 0x100) == -1                                   # logits overlap x
    assert L.moe_router_route_workspace_size(8, 256, 8) >= 4
    assert L.moe_router_route_workspace_size(100000, 256, 8) > L.moe_route_workspace_size(100000, 256, 8)


def test_stream_read_probe_argument_errors(L):
    assert L.moe_bench_stream_read(None, 0, None, None) == 0                  # nothing to read
    assert L.moe_bench_stream_read(None, 64, A + 0x4000000, None) == -1
    assert L.moe_bench_stream_read(A, 64, None, None) == -1
    assert L.moe_bench_stream_read(A, 40, A + 0x4000000, None) == -2         # not a multiple of 16
    assert L.moe_bench_stream_read(A + 8, 64, A + 0x4000000, None) == -3
    assert L.moe_bench_stream_read(A, 64, A + 0x4000002, None) == -3
