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
# throughput and one-instruction probes, and the HBM streaming probes that
# bench.py reports beside the rooflines
PROBE_SOURCES = ["mfma_probe.hip", "stream_probe.hip"]
PROBE_PATH = os.path.join(LIB_DIR, "libfp8probe.so")
# measurement support: the library again, with per-workgroup phase
# timestamps in the GEMM (bench.py --phase-timing)
PHASE_PATH = os.path.join(LIB_DIR, "libfp8phase.so")
PHASE_FLAGS = ["-DFP8L_PHASE_TIMING"]
ARCH = os.environ.get("FP8L_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=" + ARCH,
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Compile the library (every HIP source of the method) and the two
    measurement libraries, in parallel; always rebuilds."""
    os.makedirs(LIB_DIR, exist_ok=True)
    jobs = []
    for sources, out, extra in ((SOURCES, LIB_PATH, []), (PROBE_SOURCES, PROBE_PATH, []),
                                (SOURCES, PHASE_PATH, PHASE_FLAGS)):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = (["hipcc"] + HIPCC_FLAGS + extra + [os.path.join(CSRC, s) for s in sources] +
               ["-o", tmp])
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((subprocess.Popen(cmd), cmd, tmp, out))
    failed = [cmd for p, cmd, _, _ in jobs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    for _, _, tmp, out in jobs:
        os.replace(tmp, out)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
