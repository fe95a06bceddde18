"""The MFMA-only probe that bench.py reports as mfma_ceiling computes what it
is said to compute (so its flop count is right): with every code 0x38
(E4M3 1.0), each 16x16x128 MFMA adds 128 to every output element, and each
of the 8 passes of an iteration reaches every accumulator block once, so
every lane's sum of its 256 accumulators is 256 * 8 * 128 * iters.  All-zero
codes give 0.  Not part of the method: measurement support."""
import ctypes

import pytest
import torch

from float8_mixed_precision_amd import build as B
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _probe():
    L = ctypes.CDLL(B.PROBE_PATH)
    P, i64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.fp8_probe_mfma_loop.restype = I
    L.fp8_probe_mfma_loop.argtypes = [P, i64, I, I, P, P]
    return L


@pytest.mark.parametrize("iters", [1, 3])
def test_mfma_probe_counts(iters):
    L = _probe()
    wg = 4
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for code, want in ((0x38, 256.0 * 8 * 128 * iters), (0x00, 0.0)):
        codes = torch.full((1 << 17,), code, dtype=torch.uint8, device=G.DEV)
        sink = torch.full((wg * 256,), -1.0, dtype=torch.float32, device=G.DEV)
        G.say("mfma probe", hex(code), "iters", iters)
        assert L.fp8_probe_mfma_loop(codes.data_ptr(), codes.numel(), wg, iters,
                                     sink.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        assert torch.all(sink == want), (code, sink.unique()[:8])
