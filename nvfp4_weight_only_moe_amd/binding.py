"""Thin ctypes binding of libmoe_w4a16.so (C ABI in include/moe_w4a16.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device memory and the current HIP stream.  The entry points
keep the C names; each checks the returned status and raises ``MoeError``.
There is no CPU fallback: if the library is missing, loading raises.
"""

import ctypes
import os
import re
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_w4a16.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "moe_w4a16.h")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_ALIGN",
          -4: "MOE_ERR_UNSUPPORTED", -5: "MOE_ERR_NONFINITE", -6: "MOE_ERR_BAD_SCALE",
          -7: "MOE_ERR_WORKSPACE", -8: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class NVFP4TensorC(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_TP = ctypes.POINTER(NVFP4TensorC)

_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_w4a16_version": (_I, []),
    "moe_w4a16_quantize_pack": (_I, [_P, _I, _I, _I, _TP, _P]),
    "moe_w4a16_dequantize": (_I, [_TP, _P, _P]),
    "moe_w4a16_validate": (_I, [_TP, _P, _P]),
    "moe_route_workspace_size": (_S, [_I, _I, _I]),
    "moe_route_topk": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
    "moe_w4a16_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "moe_w4a16_forward": (_I, [_P, _I, _I, _I, _I, _I, _TP, _TP, _TP, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
    "moe_w4a16_route_forward": (_I, [_P, _P, _I, _I, _I, _I, _I, _TP, _TP, _TP, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _S, _P]),
    "moe_w4a16_linear_workspace_size": (_S, [_I, _I, _I]),
    "moe_w4a16_linear": (_I, [_P, _I, _I, _I, _TP, _P, _P, _S, _P]),
    "moe_router_logits": (_I, [_P, _I, _I, _P, _I, _P, _P]),
    "moe_w4a16_shared_expert_workspace_size": (_S, [_I, _I, _I]),
    "moe_w4a16_shared_expert": (_I, [_P, _I, _I, _I, _TP, _TP, _TP, _P, _P, _S, _P]),
    "moe_debug_set_prefill_variant": (_I, [_I]),
    "moe_bench_stream_read": (_I, [_P, _S, _P, _P]),
    "moe_nvfp4_quantize_activations": (_I, [_P, _I, _I, ctypes.c_float, _P, _P, _P]),
    "moe_w4a4_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "moe_w4a4_forward": (_I, [_P, _I, _I, _I, _I, _I, _TP, _TP, _TP, ctypes.c_float, ctypes.c_float,
                              _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
    "moe_w4a4_route_forward": (_I, [_P, _P, _I, _I, _I, _I, _I, _TP, _TP, _TP, ctypes.c_float, ctypes.c_float,
                                    _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
    "moe_w4a16_route_forward_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _I, _TP, _TP, _TP, _P, _P, _P, _P, _P, _P, _P,
                                             _P]),
    "moe_router_route_workspace_size": (_S, [_I, _I, _I]),
    "moe_router_route_topk": (_I, [_P, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
    "moe_profile_begin": (_I, [_I]),
    "moe_profile_end": (_I, [_P, _P, _P, _I]),
}


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_symbols():
    """Names of the functions include/moe_w4a16.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def status_string(status):
    return lib().moe_status_string(int(status)).decode()


def _check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


_BITS16 = (torch.int16, torch.uint16, torch.bfloat16) if hasattr(torch, "uint16") else (torch.int16, torch.bfloat16)


def _dev_tensor(t, name, dtype=None, shape=None, min_bytes=None):
    """The C ABI takes bare pointers and (for outputs) no sizes, so the
    binding checks every tensor before the call: a device tensor,
    contiguous, of the expected dtype(s) and exact shape (or at least
    `min_bytes`).  Raises ValueError instead of calling into the library."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a device (cuda) tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None:
        ok = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in ok:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in ok)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, at least {min_bytes} needed")
    return t


@dataclass
class NVFP4Tensor:
    """E experts of an [N, K] NVFP4 projection in canonical layout (device)."""
    codes: torch.Tensor         # uint8 [E, N, K/2]
    scales: torch.Tensor        # uint8 [E, N, K/16]
    global_scale: torch.Tensor  # float32 [E]

    @property
    def shape(self):
        E, N, half = self.codes.shape
        return E, N, half * 2

    def check(self, name="tensor"):
        E, N, K = self.shape
        _dev_tensor(self.codes, f"{name}.codes", torch.uint8, (E, N, K // 2))
        _dev_tensor(self.scales, f"{name}.scales", torch.uint8, (E, N, K // 16))
        _dev_tensor(self.global_scale, f"{name}.global_scale", torch.float32, (E,))
        return self

    def cstruct(self):
        self.check()
        E, N, K = self.shape
        return NVFP4TensorC(E, N, K, self.codes.data_ptr(), self.scales.data_ptr(),
                            self.global_scale.data_ptr())

    @staticmethod
    def empty(E, N, K, device="cuda"):
        return NVFP4Tensor(torch.empty((E, N, K // 2), dtype=torch.uint8, device=device),
                           torch.empty((E, N, K // 16), dtype=torch.uint8, device=device),
                           torch.empty((E,), dtype=torch.float32, device=device))


def moe_w4a16_version():
    return int(lib().moe_w4a16_version())


def moe_w4a16_quantize_pack(w, out=None, stream=None):
    """fp32 masters [E, N, K] (device) -> NVFP4Tensor."""
    _dev_tensor(w, "w", torch.float32)
    E, N, K = w.shape
    out = NVFP4Tensor.empty(E, N, K, w.device) if out is None else out
    if out.shape != (E, N, K):
        raise ValueError(f"out: shape {out.shape}, expected {(E, N, K)}")
    st = out.cstruct()
    _check(lib().moe_w4a16_quantize_pack(_ptr(w), E, N, K, ctypes.byref(st), _stream(stream)),
           "moe_w4a16_quantize_pack")
    return out


def moe_w4a16_dequantize(t, out=None, stream=None):
    E, N, K = t.shape
    out = torch.empty((E, N, K), dtype=torch.float32, device=t.codes.device) if out is None else out
    _dev_tensor(out, "out", torch.float32, (E, N, K))
    st = t.cstruct()
    _check(lib().moe_w4a16_dequantize(ctypes.byref(st), _ptr(out), _stream(stream)), "moe_w4a16_dequantize")
    return out


def moe_w4a16_validate(t, flag=None, stream=None):
    """Synchronises; raises MoeError on a bad scale.  `flag`: an optional
    caller-owned device tensor of at least 4 bytes (allocated here if None)."""
    flag = torch.empty((4,), dtype=torch.int32, device=t.codes.device) if flag is None else flag
    _dev_tensor(flag, "flag", min_bytes=4)
    st = t.cstruct()
    _check(lib().moe_w4a16_validate(ctypes.byref(st), _ptr(flag), _stream(stream)), "moe_w4a16_validate")


def moe_route_workspace_size(T, E, k):
    return int(lib().moe_route_workspace_size(T, E, k))


def moe_w4a16_workspace_size(T, H, I, E, k):
    return int(lib().moe_w4a16_workspace_size(T, H, I, E, k))


@dataclass
class Routing:
    topk_ids: torch.Tensor      # int32 [T, k]
    topk_w: torch.Tensor        # float32 [T, k]
    counts: torch.Tensor        # int32 [E]
    offsets: torch.Tensor       # int32 [E + 1]
    sorted_slots: torch.Tensor  # int32 [T * k]
    slot_pos: torch.Tensor      # int32 [T * k]
    ws: torch.Tensor            # uint8 workspace

    @staticmethod
    def empty(T, E, k, device="cuda"):
        i32 = dict(dtype=torch.int32, device=device)
        return Routing(torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=device),
                       torch.empty((E,), **i32), torch.empty((E + 1,), **i32),
                       torch.empty((T * k,), **i32), torch.empty((T * k,), **i32),
                       torch.empty((max(moe_route_workspace_size(T, E, k), 16),), dtype=torch.uint8,
                                   device=device))

    def check(self, T, E, k):
        i32 = torch.int32
        _dev_tensor(self.topk_ids, "routing.topk_ids", i32, (T, k))
        _dev_tensor(self.topk_w, "routing.topk_w", torch.float32, (T, k))
        _dev_tensor(self.counts, "routing.counts", i32, (E,))
        _dev_tensor(self.offsets, "routing.offsets", i32, (E + 1,))
        _dev_tensor(self.sorted_slots, "routing.sorted_slots", i32, (T * k,))
        _dev_tensor(self.slot_pos, "routing.slot_pos", i32, (T * k,))
        _dev_tensor(self.ws, "routing.ws", torch.uint8, min_bytes=moe_route_workspace_size(T, E, k))
        return self


def moe_route_topk(logits, k, out=None, stream=None):
    """fp32 logits [T, E] (device) -> Routing."""
    _dev_tensor(logits, "logits", torch.float32)
    T, E = logits.shape
    r = Routing.empty(T, E, k, logits.device) if out is None else out
    r.check(T, E, k)
    _check(lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(r.topk_ids), _ptr(r.topk_w), _ptr(r.counts),
                                _ptr(r.offsets), _ptr(r.sorted_slots), _ptr(r.slot_pos), _ptr(r.ws),
                                r.ws.numel(), _stream(stream)), "moe_route_topk")
    return r


def forward_workspace(T, H, I, E, k, device="cuda"):
    """A forward workspace (needs no initialisation)."""
    return torch.empty((max(moe_w4a16_workspace_size(T, H, I, E, k), 256),), dtype=torch.uint8, device=device)


def moe_bench_stream_read(src, nbytes, sink, stream=None):
    """Stream-read the first nbytes of the device tensor src (a benchmark
    reference; see the header); sink: a device int32/uint32 tensor of >= 1
    element."""
    _dev_tensor(src, "src", min_bytes=nbytes)
    _dev_tensor(sink, "sink", min_bytes=4)
    _check(lib().moe_bench_stream_read(_ptr(src), int(nbytes), _ptr(sink), _stream(stream)), "moe_bench_stream_read")


def moe_debug_set_prefill_variant(variant):
    _check(lib().moe_debug_set_prefill_variant(int(variant)), "moe_debug_set_prefill_variant")


def moe_w4a16_forward(x_bits, gate, up, down, routing, out=None, ws=None, stream=None):
    """bf16 activations (int16/uint16 bit patterns or torch.bfloat16) [T, H] ->
    bf16 bits [T, H] (int16 tensor; view as torch.bfloat16 for values)."""
    _dev_tensor(x_bits, "x", _BITS16)
    T, H = x_bits.shape
    E, I, _ = gate.shape
    k = routing.topk_ids.shape[1]
    routing.check(T, E, k)
    out = torch.empty((T, H), dtype=torch.int16, device=x_bits.device) if out is None else out
    _dev_tensor(out, "out", _BITS16, (T, H))
    ws = forward_workspace(T, H, I, E, k, x_bits.device) if ws is None else ws
    _dev_tensor(ws, "ws", min_bytes=moe_w4a16_workspace_size(T, H, I, E, k))
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    _check(lib().moe_w4a16_forward(_ptr(x_bits), T, H, I, E, k, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                   _ptr(routing.topk_ids), _ptr(routing.topk_w), _ptr(routing.counts),
                                   _ptr(routing.offsets), _ptr(routing.sorted_slots), _ptr(routing.slot_pos),
                                   _ptr(out), _ptr(ws), ws.numel(), _stream(stream)), "moe_w4a16_forward")
    return out


def moe_w4a16_route_forward(logits, x_bits, gate, up, down, k, routing=None, out=None, ws=None, stream=None):
    """Route (as moe_route_topk, outputs stored in `routing`) and run the
    layer (with one token the gate/up kernel routes itself).  Returns
    (out, routing)."""
    _dev_tensor(x_bits, "x", _BITS16)
    T, H = x_bits.shape
    E, I, _ = gate.shape
    _dev_tensor(logits, "logits", torch.float32, (T, E))
    routing = Routing.empty(T, E, k, x_bits.device) if routing is None else routing
    routing.check(T, E, k)
    out = torch.empty((T, H), dtype=torch.int16, device=x_bits.device) if out is None else out
    _dev_tensor(out, "out", _BITS16, (T, H))
    ws = forward_workspace(T, H, I, E, k, x_bits.device) if ws is None else ws
    _dev_tensor(ws, "ws", min_bytes=moe_w4a16_workspace_size(T, H, I, E, k))
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    _check(lib().moe_w4a16_route_forward(_ptr(logits), _ptr(x_bits), T, H, I, E, k, ctypes.byref(g), ctypes.byref(u),
                                         ctypes.byref(d), _ptr(routing.topk_ids), _ptr(routing.topk_w),
                                         _ptr(routing.counts), _ptr(routing.offsets), _ptr(routing.sorted_slots),
                                         _ptr(routing.slot_pos), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_w4a16_route_forward")
    return out, routing


def moe_profile_begin(max_launches=4096):
    _check(lib().moe_profile_begin(max_launches), "moe_profile_begin")


def moe_profile_end(max_names=64):
    """Synchronises; returns {kernel name: (launches, total ms)}."""
    names = (ctypes.c_char * 64 * max_names)()
    counts = (ctypes.c_int32 * max_names)()
    ms = (ctypes.c_double * max_names)()
    n = lib().moe_profile_end(ctypes.cast(names, ctypes.c_void_p), ctypes.cast(counts, ctypes.c_void_p),
                              ctypes.cast(ms, ctypes.c_void_p), max_names)
    return {names[i].value.decode(): (int(counts[i]), float(ms[i])) for i in range(n)}


def moe_router_logits(x_bits, wr_bits, out=None, stream=None):
    """Router logits: bf16 bits x [T, H] and router weight [E, H] (int16
    tensors) -> fp32 [T, E]."""
    _dev_tensor(x_bits, "x", _BITS16)
    _dev_tensor(wr_bits, "wr", _BITS16)
    T, H = x_bits.shape
    E, H2 = wr_bits.shape
    if H2 != H:
        raise ValueError(f"wr: {H2} columns, x has {H}")
    out = torch.empty((T, E), dtype=torch.float32, device=x_bits.device) if out is None else out
    _dev_tensor(out, "out", torch.float32, (T, E))
    _check(lib().moe_router_logits(_ptr(x_bits), T, H, _ptr(wr_bits), E, _ptr(out), _stream(stream)),
           "moe_router_logits")
    return out


def moe_w4a16_linear(x_bits, w, out=None, ws=None, stream=None):
    """Dense projection: bf16 bits [T, K] and an NVFP4 tensor with E = 1,
    shape [1, N, K] -> bf16 bits [T, N] (int16 tensor)."""
    _dev_tensor(x_bits, "x", _BITS16)
    T, K = x_bits.shape
    E, N, K2 = w.shape
    if E != 1 or K2 != K:
        raise ValueError(f"w: shape {(E, N, K2)}, expected (1, N, {K})")
    out = torch.empty((T, N), dtype=torch.int16, device=x_bits.device) if out is None else out
    _dev_tensor(out, "out", _BITS16, (T, N))
    if ws is None:
        ws = torch.empty((max(lib().moe_w4a16_linear_workspace_size(max(T, 1), K, N), 256),), dtype=torch.uint8,
                         device=x_bits.device)
    _dev_tensor(ws, "ws", min_bytes=lib().moe_w4a16_linear_workspace_size(T, K, N))
    c = w.cstruct()
    _check(lib().moe_w4a16_linear(_ptr(x_bits), T, K, N, ctypes.byref(c), _ptr(out), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_w4a16_linear")
    return out


def moe_w4a16_shared_expert(x_bits, gate, up, down, out=None, ws=None, stream=None):
    """The shared expert (one SwiGLU FFN for every token): bf16 bits [T, H]
    and NVFP4 tensors with E = 1 -> bf16 bits [T, H] (int16 tensor)."""
    _dev_tensor(x_bits, "x", _BITS16)
    T, H = x_bits.shape
    E, I, _ = gate.shape
    if E != 1:
        raise ValueError(f"gate: {E} experts, the shared expert has 1")
    out = torch.empty((T, H), dtype=torch.int16, device=x_bits.device) if out is None else out
    _dev_tensor(out, "out", _BITS16, (T, H))
    if ws is None:
        ws = torch.empty((max(lib().moe_w4a16_shared_expert_workspace_size(max(T, 1), H, I), 256),),
                         dtype=torch.uint8, device=x_bits.device)
    _dev_tensor(ws, "ws", min_bytes=lib().moe_w4a16_shared_expert_workspace_size(T, H, I))
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    _check(lib().moe_w4a16_shared_expert(_ptr(x_bits), T, H, I, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                         _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_w4a16_shared_expert")
    return out


def _input_scale(s, name):
    """A W4A4 input scale as a Python float; None (a missing scale) is
    refused here, everything else is checked by the library."""
    if s is None:
        raise ValueError(f"{name} is missing: a W4A4 layer needs its static input scale")
    return float(s)


def moe_nvfp4_quantize_activations(x_bits, input_scale, codes=None, scales=None, stream=None):
    """bf16 bits [T, K] -> (codes uint8 [T, K/2], scales uint8 [T, K/16])."""
    s = _input_scale(input_scale, "input_scale")
    _dev_tensor(x_bits, "x", _BITS16)
    T, K = x_bits.shape
    codes = torch.empty((T, K // 2), dtype=torch.uint8, device=x_bits.device) if codes is None else codes
    scales = torch.empty((T, K // 16), dtype=torch.uint8, device=x_bits.device) if scales is None else scales
    _dev_tensor(codes, "codes", torch.uint8, (T, K // 2))
    _dev_tensor(scales, "scales", torch.uint8, (T, K // 16))
    _check(lib().moe_nvfp4_quantize_activations(_ptr(x_bits), T, K, s, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_nvfp4_quantize_activations")
    return codes, scales


def moe_w4a4_workspace_size(T, H, I, E, k):
    return int(lib().moe_w4a4_workspace_size(T, H, I, E, k))


def moe_w4a4_forward(x_bits, gate, up, down, routing, input_scale_x, input_scale_h, out=None, ws=None,
                     stream=None):
    """The W4A4 layer: bf16 bits [T, H] -> bf16 bits [T, H] (int16 tensor)."""
    sx = _input_scale(input_scale_x, "input_scale_x")
    sh = _input_scale(input_scale_h, "input_scale_h")
    _dev_tensor(x_bits, "x", _BITS16)
    T, H = x_bits.shape
    E, I, _ = gate.shape
    k = routing.topk_ids.shape[1]
    routing.check(T, E, k)
    out = torch.empty((T, H), dtype=torch.int16, device=x_bits.device) if out is None else out
    _dev_tensor(out, "out", _BITS16, (T, H))
    need = moe_w4a4_workspace_size(T, H, I, E, k)
    ws = torch.empty((max(need, 256),), dtype=torch.uint8, device=x_bits.device) if ws is None else ws
    _dev_tensor(ws, "ws", min_bytes=need)
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    _check(lib().moe_w4a4_forward(_ptr(x_bits), T, H, I, E, k, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                  sx, sh, _ptr(routing.topk_ids), _ptr(routing.topk_w), _ptr(routing.counts),
                                  _ptr(routing.offsets), _ptr(routing.sorted_slots), _ptr(routing.slot_pos),
                                  _ptr(out), _ptr(ws), ws.numel(), _stream(stream)), "moe_w4a4_forward")
    return out


def moe_w4a4_route_forward(logits, x_bits, gate, up, down, k, input_scale_x, input_scale_h, routing=None,
                           out=None, ws=None, stream=None):
    """Route (as moe_route_topk, outputs stored in `routing`) and run the W4A4
    layer (with one token the gate/up kernel routes itself).  Returns
    (out, routing)."""
    sx = _input_scale(input_scale_x, "input_scale_x")
    sh = _input_scale(input_scale_h, "input_scale_h")
    _dev_tensor(x_bits, "x", _BITS16)
    T, H = x_bits.shape
    E, I, _ = gate.shape
    _dev_tensor(logits, "logits", torch.float32, (T, E))
    routing = Routing.empty(T, E, k, x_bits.device) if routing is None else routing
    routing.check(T, E, k)
    out = torch.empty((T, H), dtype=torch.int16, device=x_bits.device) if out is None else out
    _dev_tensor(out, "out", _BITS16, (T, H))
    need = moe_w4a4_workspace_size(T, H, I, E, k)
    ws = torch.empty((max(need, 256),), dtype=torch.uint8, device=x_bits.device) if ws is None else ws
    _dev_tensor(ws, "ws", min_bytes=need)
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    _check(lib().moe_w4a4_route_forward(_ptr(logits), _ptr(x_bits), T, H, I, E, k, ctypes.byref(g), ctypes.byref(u),
                                        ctypes.byref(d), sx, sh, _ptr(routing.topk_ids), _ptr(routing.topk_w),
                                        _ptr(routing.counts), _ptr(routing.offsets), _ptr(routing.sorted_slots),
                                        _ptr(routing.slot_pos), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_w4a4_route_forward")
    return out, routing


def moe_w4a16_route_forward_noalloc(logits, x_bits, gate, up, down, k, routing=None, out=None, stream=None):
    """moe_w4a16_route_forward with the library's own device array as the
    workspace (no workspace argument, no allocation in the call).  Returns
    (out, routing)."""
    _dev_tensor(x_bits, "x", _BITS16)
    T, H = x_bits.shape
    E, I, _ = gate.shape
    _dev_tensor(logits, "logits", torch.float32, (T, E))
    routing = Routing.empty(T, E, k, x_bits.device) if routing is None else routing
    routing.check(T, E, k)
    out = torch.empty((T, H), dtype=torch.int16, device=x_bits.device) if out is None else out
    _dev_tensor(out, "out", _BITS16, (T, H))
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    _check(lib().moe_w4a16_route_forward_noalloc(_ptr(logits), _ptr(x_bits), T, H, I, E, k, ctypes.byref(g),
                                                 ctypes.byref(u), ctypes.byref(d), _ptr(routing.topk_ids),
                                                 _ptr(routing.topk_w), _ptr(routing.counts), _ptr(routing.offsets),
                                                 _ptr(routing.sorted_slots), _ptr(routing.slot_pos), _ptr(out),
                                                 _stream(stream)), "moe_w4a16_route_forward_noalloc")
    return out, routing


def router_route_workspace(T, E, k, device="cuda"):
    """A workspace for moe_router_route_topk, zero-filled (its ticket word
    must start at zero; every call leaves it zero)."""
    n = int(lib().moe_router_route_workspace_size(T, E, k))
    return torch.zeros((max(n, 256),), dtype=torch.uint8, device=device)


def moe_router_route_topk(x_bits, wr_bits, k, logits=None, routing=None, ws=None, stream=None):
    """Router logits and the route in one call: bf16 bits x [T, H], router
    weight [E, H] -> (fp32 logits [T, E], Routing)."""
    _dev_tensor(x_bits, "x", _BITS16)
    _dev_tensor(wr_bits, "wr", _BITS16)
    T, H = x_bits.shape
    E, H2 = wr_bits.shape
    if H2 != H:
        raise ValueError(f"wr: {H2} columns, x has {H}")
    logits = torch.empty((T, E), dtype=torch.float32, device=x_bits.device) if logits is None else logits
    _dev_tensor(logits, "logits", torch.float32, (T, E))
    routing = Routing.empty(T, E, k, x_bits.device) if routing is None else routing
    routing.check(T, E, k)
    ws = router_route_workspace(T, E, k, x_bits.device) if ws is None else ws
    _dev_tensor(ws, "ws", min_bytes=int(lib().moe_router_route_workspace_size(T, E, k)))
    _check(lib().moe_router_route_topk(_ptr(x_bits), T, H, _ptr(wr_bits), E, k, _ptr(logits), _ptr(routing.topk_ids),
                                       _ptr(routing.topk_w), _ptr(routing.counts), _ptr(routing.offsets),
                                       _ptr(routing.sorted_slots), _ptr(routing.slot_pos), _ptr(ws), ws.numel(),
                                       _stream(stream)), "moe_router_route_topk")
    return logits, routing
