"""fp8_linear_quantize_noalloc (no workspace argument; the library's per-GPU
scratch array) gives fp8_linear_quantize's results bit for bit, on two calls
in a row, the second with a smaller input, in both scalings and both code
formats; the scratch array keeps the first call's contents, which the
second call must not depend on."""
import numpy as np
import pytest
import torch

from float8_mixed_precision_amd import ops
from float8_mixed_precision_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("e5m2", [False, True], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_noalloc_equals_quantize(rowwise, e5m2):
    for n, (rows, cols) in enumerate(((4096, 8208), (272, 400))):
        x = G.dev_bf16(W.random_bf16(90 + n, (rows, cols), 1.0 if n else 3.0, int(rowwise)))
        G.say("noalloc quantize", (rows, cols), "rowwise", rowwise, "e5m2", e5m2)
        ref = ops.fp8_linear_quantize(x, rowwise, e5m2=e5m2)
        out = ops.alloc_quantized(rows, cols, rowwise, x.device)
        for t in (out.q, out.qt):
            t.fill_(0xA5)
        for t in (out.scale, out.scale_t, out.amax):
            t.fill_(-1.0)
        ops.fp8_linear_quantize_noalloc(x, rowwise, out=out, e5m2=e5m2)
        torch.cuda.synchronize()
        got = (G.host(out.q), G.host(out.qt), G.host(out.scale), G.host(out.scale_t),
               G.host(out.amax))
        want = (G.host(ref.q), G.host(ref.qt), G.host(ref.scale), G.host(ref.scale_t),
                G.host(ref.amax))
        G.assert_quantize_equal(got, want, "noalloc %s" % ((rows, cols),))
