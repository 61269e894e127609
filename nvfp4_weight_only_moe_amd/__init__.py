"""NVFP4 weight-only (W4A16) routed-expert MoE layer for AMD MI355X (gfx950).

The compute lives in the HIP shared library ``libmoe_w4a16.so`` behind the C
ABI declared in ``include/moe_w4a16.h``; ``nvfp4_weight_only_moe_amd.binding``
is a thin ctypes layer with the same entry-point names.  Importing this
package loads nothing; the binding loads the library on first use and raises
if it is missing -- there is no CPU fallback.
"""

__all__ = ["binding", "workloads"]
