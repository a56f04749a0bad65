"""Build libmoe_dc.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every translation unit is compiled by hipcc with floating-point contraction off (each written
float operation stays one IEEE operation), IEEE division, fp32 subnormals kept, and the
packed-FP32 instructions disabled.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_dc.so")
SOURCES = ["api.cpp", "route.hip", "dispatch.hip", "combine.hip", "noalloc.hip"]
# measurement kernels of bench.py's ceiling mode (the access patterns without the arithmetic)
CEILING_LIB = os.path.join(HERE, "libmoe_dc_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
# exhaustive GPU checks of the instruction-level conversions, for the tests
SELFCHECK_LIB = os.path.join(HERE, "libmoe_dc_selfcheck.so")
SELFCHECK_SOURCES = ["selfcheck.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror",
    "-ffp-contract=off", "-fno-fast-math",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]
DEVICE = [
    f"--offload-arch={ARCH}", "-fno-gpu-rdc",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source, link libmoe_dc.so, the ceiling-measurement library and the
    conversion self-check library; returns the path of libmoe_dc.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES + SELFCHECK_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    n, c = len(SOURCES), len(CEILING_SOURCES)
    _link(objs[:n], LIB, verbose)
    _link(objs[n:n + c], CEILING_LIB, verbose)
    _link(objs[n + c:], SELFCHECK_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
