"""Helpers for the GPU parity tests (not a test module).

Inputs come from nvfp4_weight_only_moe_amd.workloads; expected values come
from the oracle alone, which quantizes the same seeded masters itself.  The
HIP path is driven only through the C ABI (nvfp4_weight_only_moe_amd.binding).
"""
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from oracle import moe as omoe
from nvfp4_weight_only_moe_amd import binding as B
from nvfp4_weight_only_moe_amd import workloads as wls

DEV = "cuda:0"
PROJ = ((wls.GATE, "gate"), (wls.UP, "up"), (wls.DOWN, "down"))
THREADS = min(16, os.cpu_count() or 4)

# Output parity bar: relative Frobenius error and per-element error relative
# to the largest reference magnitude.
REL_FRO = 5e-3
REL_MAX = 1e-2


def log(msg):
    print(f"[gpu-test {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def bf16_bits_to_f64(t):
    """int16 tensor of bf16 bits -> float64 numpy."""
    return t.view(torch.bfloat16).to(torch.float64).cpu().numpy()


def compare_out(got, ref, where=""):
    """Assert the layer-output bar; returns (rel_fro, rel_max, cosine, norm_ratio)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{where}: non-finite output"
    nref = np.linalg.norm(ref)
    rel_fro = float(np.linalg.norm(got - ref) / max(nref, 1e-300))
    rel_max = float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300)) if ref.size else 0.0
    cos = float((got * ref).sum() / max(np.linalg.norm(got) * nref, 1e-300))
    ratio = float(np.linalg.norm(got) / max(nref, 1e-300))
    log(f"{where}: rel_fro={rel_fro:.3e} rel_max={rel_max:.3e} cos={cos:.7f} norm_ratio={ratio:.5f}")
    assert rel_fro <= REL_FRO, (where, rel_fro)
    assert rel_max <= REL_MAX, (where, rel_max)
    return rel_fro, rel_max, cos, ratio


# ------------------------------------------------------------------ guard bands
GUARD_BYTES = 4096
GUARD_BYTE = 0xA5


class Guarded:
    """A device buffer between two guard bands of GUARD_BYTES filled with a
    byte pattern; ``t`` is the caller-visible tensor (contiguous, 256-byte
    aligned).  ``check`` asserts both bands, and the padding up to the next
    256-byte boundary, still hold the pattern after the library wrote ``t``:
    every kernel writes through computed indices, so a stray write shows up
    here even when it lands where no parity check looks."""

    def __init__(self, shape, dtype, device=DEV):
        shape = tuple(int(d) for d in shape)
        nbytes = int(np.prod(shape, dtype=np.int64)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = nbytes
        padded = (nbytes + 255) // 256 * 256
        self.raw = torch.full((GUARD_BYTES + padded + GUARD_BYTES,), GUARD_BYTE, dtype=torch.uint8, device=device)
        self.t = self.raw[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(shape)

    def check(self, where):
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[GUARD_BYTES + self.nbytes:]
        bad_head = int((head != GUARD_BYTE).sum())
        bad_tail = int((tail != GUARD_BYTE).sum())
        assert bad_head == 0 and bad_tail == 0, f"{where}: {bad_head} guard bytes before and {bad_tail} after changed"


def guarded_routing(T, E, k):
    """A Routing whose every array (and route scratch) sits between guard bands."""
    parts = {
        "topk_ids": Guarded((T, k), torch.int32), "topk_w": Guarded((T, k), torch.float32),
        "counts": Guarded((E,), torch.int32), "offsets": Guarded((E + 1,), torch.int32),
        "sorted_slots": Guarded((T * k,), torch.int32), "slot_pos": Guarded((T * k,), torch.int32),
        "ws": Guarded((max(B.moe_route_workspace_size(T, E, k), 16),), torch.uint8),
    }
    r = B.Routing(**{n: g.t for n, g in parts.items()})
    return r, parts


def check_guards(parts, where):
    for name, g in parts.items():
        g.check(f"{where}: {name}")


def guarded_forward(x_bits, gate, up, down, logits, k, fused):
    """Route + forward (two calls, or moe_w4a16_route_forward when `fused`)
    into guarded output, routing and workspace buffers sized exactly as the
    header states; asserts the guards and returns (out, routing)."""
    T, H = x_bits.shape
    E, I, _ = gate.shape
    r, parts = guarded_routing(T, E, k)
    parts["out"] = Guarded((T, H), torch.int16)
    parts["forward_ws"] = Guarded((max(B.moe_w4a16_workspace_size(T, H, I, E, k), 16),), torch.uint8)
    out, ws = parts["out"].t, parts["forward_ws"].t
    if fused:
        B.moe_w4a16_route_forward(logits, x_bits, gate, up, down, k, routing=r, out=out, ws=ws)
    else:
        B.moe_route_topk(logits, k, out=r)
        B.moe_w4a16_forward(x_bits, gate, up, down, r, out=out, ws=ws)
    torch.cuda.synchronize()
    check_guards(parts, f"T{T} H{H} I{I} E{E} k{k} {'route_forward' if fused else 'route+forward'}")
    return out, r


# ------------------------------------------------------------------ packing
def pack_gpu(masters):
    """numpy fp32 [E, N, K] -> NVFP4Tensor packed by the HIP library."""
    w = to_dev(masters)
    t = B.moe_w4a16_quantize_pack(w)
    torch.cuda.synchronize()
    return t


def packed_to_numpy(t):
    return (t.codes.cpu().numpy(), t.scales.cpu().numpy(), t.global_scale.cpu().numpy())


def oracle_layer_from_masters(ms):
    """Packed oracle layer dict from a list of three [E, N, K] master stacks."""
    return {name: oracle.quantize_layer(m) for (_, name), m in zip(PROJ, ms)}


# ------------------------------------------------------------------ problems
class Problem:
    """Small seeded problem, fully computed by the oracle."""

    def __init__(self, T, H, I, E, k, seed, logits=None):
        self.wl, self.ms, self.xb, self.x, lg = wls.random_problem(seed, T, H, I, E, k)
        self.logits = lg if logits is None else logits.astype(np.float32)
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.layer = oracle_layer_from_masters(self.ms)
        self.ids, self.w = oracle.route_topk(self.logits, k) if T else (np.zeros((0, k), np.int32), np.zeros((0, k)))

    def reference(self, **kw):
        return omoe.moe_forward(self.x, self.layer, self.ids, self.w, **kw)

    def run_gpu(self, fused=False):
        """Pack on the GPU, then route + forward into guarded buffers."""
        gate, up, down = (pack_gpu(m) for m in self.ms)
        out, r = guarded_forward(to_dev(self.xb, torch.int16), gate, up, down, to_dev(self.logits), self.k, fused)
        return out, r, (gate, up, down)


# ------------------------------------------------------------------ full size
_FULL = {}


def full_layer_gpu():
    """The full-size shared layer (H=5120, I=1536, E=256) packed on the GPU;
    masters are generated on the host in batches and quantized by the HIP
    library.  Cached for the session."""
    if "gpu" in _FULL:
        return _FULL["gpu"]
    wl = wls.WORKLOADS[1]
    t0 = time.time()
    packed = {}
    for proj, name in PROJ:
        n, k = wls.proj_shape(wl, proj)
        t = B.NVFP4Tensor.empty(wl.E, n, k, DEV)
        batch = 32
        with ThreadPoolExecutor(THREADS) as ex:
            for e0 in range(0, wl.E, batch):
                ms = np.stack(list(ex.map(lambda e: wls.master(wl, proj, e), range(e0, e0 + batch))))
                w = to_dev(ms)
                sl = B.NVFP4Tensor(t.codes[e0:e0 + batch], t.scales[e0:e0 + batch], t.global_scale[e0:e0 + batch])
                B.moe_w4a16_quantize_pack(w, out=sl)
                del w
        torch.cuda.synchronize()
        packed[name] = t
        log(f"full layer: {name} packed ({time.time() - t0:.1f} s)")
    _FULL["gpu"] = packed
    return packed


def oracle_forward_parallel(x, layer, ids, w, tokens):
    """oracle.moe_forward restricted to `tokens`, with the experts' work
    (dequantize + fp64 FFN) spread over threads and the contributions then
    added in ascending expert order, as moe_forward adds them: the same
    oracle arithmetic, faster on a many-core host."""
    x = np.asarray(x, np.float64)
    ids = np.asarray(ids)
    w = np.asarray(w, np.float64)
    tokens = np.asarray(sorted(set(int(t) for t in tokens)))
    experts = [int(e) for e in np.unique(ids[tokens].reshape(-1))]

    def one(e):
        rows, slots = np.nonzero(ids[tokens] == e)
        toks = tokens[rows]
        wg, wu, wd = omoe.dequantize_expert(layer, e)
        return toks, w[toks, slots][:, None] * omoe.expert_ffn(x[toks], wg, wu, wd)

    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(one, experts))
    out = np.zeros_like(x)
    for toks, contrib in parts:
        out[toks] += contrib
    return out


_ORACLE_EXPERTS = {}


def oracle_experts(experts):
    """Oracle-packed (codes, scales, g) per (projection, expert), quantized
    from freshly generated masters; cached."""
    wl = wls.WORKLOADS[1]
    todo = [(proj, name, int(e)) for proj, name in PROJ for e in experts if (name, int(e)) not in _ORACLE_EXPERTS]
    if todo:
        t0 = time.time()
        with ThreadPoolExecutor(THREADS) as ex:
            res = list(ex.map(lambda a: oracle.quantize(wls.master(wl, a[0], a[2])), todo))
        for (proj, name, e), r in zip(todo, res):
            _ORACLE_EXPERTS[(name, e)] = r
        log(f"oracle quantized {len(todo)} tensors ({time.time() - t0:.1f} s)")
    layer = {}
    for _, name in PROJ:
        layer[name] = ({e: _ORACLE_EXPERTS[(name, int(e))][0] for e in experts},
                       {e: _ORACLE_EXPERTS[(name, int(e))][1] for e in experts},
                       {e: _ORACLE_EXPERTS[(name, int(e))][2] for e in experts})
    return layer
