"""Build the gfx950 HIP library libfp8linear.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libfp8linear.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "swiglu.hip"]
# measurement support, kept out of the method's library: the MFMA-only
# throughput probe that bench.py reports beside the GEMM's roofline
PROBE_SOURCES = ["mfma_probe.hip"]
PROBE_PATH = os.path.join(LIB_DIR, "libfp8probe.so")
ARCH = os.environ.get("FP8L_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=" + ARCH,
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
]


def _hipcc(sources, out: str, verbose: bool) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["hipcc"] + HIPCC_FLAGS + [os.path.join(CSRC, s) for s in sources] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile the library (every HIP source of the method) and the MFMA
    probe library; always rebuilds."""
    os.makedirs(LIB_DIR, exist_ok=True)
    _hipcc(SOURCES, LIB_PATH, verbose)
    _hipcc(PROBE_SOURCES, PROBE_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
