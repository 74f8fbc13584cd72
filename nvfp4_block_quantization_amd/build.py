"""Build libnvfp4.so (gfx950) in-tree with hipcc: the quantization kernels
(csrc/nvfp4.hip) and the FP4 GEMM consumer (csrc/gemm.hip); and the
measurement companion libnvfp4_membench.so (csrc/membench.hip, HBM stream
ceilings)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "nvfp4.hip"), os.path.join(HERE, "csrc", "gemm.hip")]
LIB = os.path.join(HERE, "libnvfp4.so")
MEMBENCH_SOURCES = [os.path.join(HERE, "csrc", "membench.hip")]
MEMBENCH_LIB = os.path.join(HERE, "libnvfp4_membench.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: every binary32 operation rounds on its own (no fused multiply-add),
#   which the fixed operation order of the method relies on.
# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc(sources: list, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *sources]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _hipcc(MEMBENCH_SOURCES, MEMBENCH_LIB, verbose)
    return _hipcc(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
