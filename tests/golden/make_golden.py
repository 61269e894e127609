"""Write tests/golden/tiny_layer_oracle.json from the oracle alone.

The pages print no worked example of NVFP4 packing or of the MoE layer, so
the stored values here are the oracle's own answers on the tiny seeded
workload (16 tokens, hidden 256, intermediate 128, 8 experts, top-2).  They
guard the oracle against accidental change: a later edit of its arithmetic
must regenerate this file and say, in its commit message, which passage or
reading justifies the change.  This script imports only ``oracle`` and the
seeded input generators.

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from nvfp4_weight_only_moe_amd import workloads as wls  # noqa: E402


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def build():
    wl = wls.WORKLOADS[0]
    doc = {"workload": wl.name, "projections": {}}
    layer = {}
    for proj, name in ((wls.GATE, "gate"), (wls.UP, "up"), (wls.DOWN, "down")):
        codes, scales, g = oracle.quantize_layer(wls.masters(wl, proj))
        layer[name] = (codes, scales, g)
        doc["projections"][name] = {
            "codes_sha256": sha(codes), "scales_sha256": sha(scales),
            "global_scale_hex": [float(v).hex() for v in g],
        }
    _, x = wls.activations(wl)
    lg = wls.logits(wl)
    ids, w = oracle.route_topk(lg, wl.k)
    counts, offsets, sorted_slots, slot_pos = oracle.permutation(ids, wl.E)
    out = oracle.moe_forward(x, layer, ids, w)
    doc["route"] = {"ids": ids.tolist(), "weights_hex": [[float(v).hex() for v in r] for r in w],
                    "counts": counts.tolist(), "sorted_slots": sorted_slots.tolist()}
    doc["out_rows_0_and_15_first8_hex"] = [[float(v).hex() for v in out[t, :8]] for t in (0, 15)]
    doc["out_frobenius"] = float(np.linalg.norm(out))
    return doc


if __name__ == "__main__":
    path = os.path.join(HERE, "tiny_layer_oracle.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=1)
    print("wrote", path)
