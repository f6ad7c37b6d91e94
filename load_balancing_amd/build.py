"""Build libmoonep.so and libmoonep_ceilings.so (gfx950) in-tree with hipcc.

    python -m load_balancing_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoonep.so")
SOURCES = ["abi.hip", "route_stats.hip", "plan.hip", "movers.hip", "reduce.hip", "prefetch.hip", "gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Plain IEEE arithmetic in source order; fused multiply-adds are written out.
    "-ffp-contract=off",
    # No packed fp32 instructions: scalar or float2 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# The machine-ceiling microbenchmarks (bench.py --ceilings): a library of
# their own, outside libmoonep's C-ABI.
CEIL_LIB = os.path.join(HERE, "libmoonep_ceilings.so")
CEIL_SOURCES = ["ceilings.hip"]


def _hipcc(sources, out, verbose):
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    """The ceilings library, then libmoonep.so; returns the path of libmoonep.so."""
    _hipcc(CEIL_SOURCES, CEIL_LIB, verbose)
    return _hipcc(SOURCES, LIB, verbose)


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
