"""Build libmoe_w4a16.so (gfx950) in-tree with hipcc.

    python -m nvfp4_weight_only_moe_amd.build_lib      # or build() from Python

Every source in csrc/ is compiled to an object under csrc/_build/ (in
parallel) and linked into nvfp4_weight_only_moe_amd/libmoe_w4a16.so.  Flags:

* ``--offload-arch=gfx950`` only: the kernels use gfx950 instructions
  (FP4 conversion, 16x16x32 bf16 MFMA) and there is no other target;
* packed-fp32 instructions are disabled (``-packed-fp32-ops``): hipcc would
  otherwise form them from ordinary float code;
* fp32 division and square root are correctly rounded and fp32 denormals are
  kept: the quantizer must reproduce the exact fp32 scale arithmetic.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "libmoe_w4a16.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SOURCES = ["abi.cpp", "quantize.hip", "route.hip", "moe_decode.hip", "moe_prefill.hip", "moe_prefill_pipe.hip",
           "router.hip", "noalloc.hip", "probe.hip"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says
    # so; that warning is expected and dropped here.
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose=False, jobs=None):
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


ASAN_LIB = os.path.join(BUILD, "libmoe_w4a16_asan.so")


CLANGXX = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang++")


def asan_runtime():
    """Path of the host compiler's AddressSanitizer runtime (to preload)."""
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_asan():
    """A copy of the library whose host code -- the C ABI's argument checking
    and dispatch, abi.cpp, which holds no device code -- is compiled as plain
    C++ by the host compiler with AddressSanitizer; every other object is the
    normal build's.  For the CPU tests of the C ABI under ASan (the runtime is
    preloaded into that test's process).  Returns its path."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o")) for s in SOURCES):
        build()
    obj = os.path.join(BUILD, "abi_asan.o")
    cmd = [CLANGXX, "-std=c++17", "-O1", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{INCLUDE}",
           f"-I{CSRC}", "-fsanitize=address", "-fno-omit-frame-pointer", "-c", os.path.join(CSRC, "abi.cpp"),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"clang++ (ASan) failed for abi.cpp:\n{r.stderr}")
    objs = [obj] + [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "abi.cpp"]
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", ASAN_LIB],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (ASan) failed:\n{r.stdout}{r.stderr}")
    return ASAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
