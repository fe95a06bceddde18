"""The whole fp8 linear (quantize X, W, dY; fwd; grad_X; grad_W) at the
workload sizes, in the launch sequence the benchmark times (LinearStep).

Quantize outputs are compared with the oracle in full, bit for bit.  GEMM
outputs are compared in full for the tiny workload and, at the full Llama
sizes, on sampled positions (random ones plus every tile boundary and the
last row / column) that the oracle computes one by one."""
import numpy as np
import pytest
import torch

import oracle
from float8_mixed_precision_amd import ops
from float8_mixed_precision_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def check_linear(lin, data, rowwise, sampled, seed):
    M, N, K = lin.M, lin.N, lin.K
    G.say("linear", lin.name, (M, N, K), "rowwise", rowwise, "upload")
    step = ops.LinearStep(G.dev_bf16(data["x"]), G.dev_bf16(data["w"]),
                          G.dev_bf16(data["dy"]), rowwise)
    G.say("linear", lin.name, "run")
    step.run()
    torch.cuda.synchronize()
    G.say("linear", lin.name, "compare quantize")
    ref = {}
    for name, qz in (("x", step.qx), ("w", step.qw), ("dy", step.qdy)):
        r = oracle.quantize(data[name], rowwise)
        got = (G.host(qz.q), G.host(qz.qt), G.host(qz.scale), G.host(qz.scale_t),
               G.host(qz.amax))
        G.assert_quantize_equal(got, r, "%s quantize %s" % (lin.name, name))
        ref[name] = r
    ox, ow, ody = ref["x"], ref["w"], ref["dy"]
    gemms = (("fwd", step.out, ox[0], ox[2], ow[0], ow[2]),
             ("grad_x", step.grad_x, ody[0], ody[2], ow[1], ow[3]),
             ("grad_w", step.grad_w, ody[1], ody[3], ox[1], ox[3]))
    for name, out_t, a, sa, b, sb in gemms:
        m, n = a.shape[0], b.shape[0]
        G.say("linear", lin.name, "compare", name, (m, n, a.shape[1]))
        if sampled:
            ii, jj = G.sample_indices(m, n, 6000, seed)
            got = G.host(out_t[torch.from_numpy(ii).to(G.DEV), torch.from_numpy(jj).to(G.DEV)])
            want = oracle.gemm_tn_sampled(a, sa, b, sb, ii, jj)
            G.gemm_parity(got, want, a, b, sa, sb, ii, jj, label="%s %s" % (lin.name, name))
        else:
            G.gemm_parity(G.host(out_t), oracle.gemm_tn(a, sa, b, sb), a, b, sa, sb,
                          label="%s %s" % (lin.name, name))
    del step
    torch.cuda.empty_cache()


def test_tiny_workload_full():
    wl = W.WORKLOADS["tiny_tw"]
    data = W.generate(wl)
    for lin, d in zip(wl.linears, data):
        check_linear(lin, d, wl.rowwise, sampled=False, seed=0)


FULL = [("attn8b_tw", 0), ("ffn8b_tw", 0), ("ffn8b_tw", 2), ("ffn70b_tw", 0), ("outlier_rw", 0)]


@pytest.mark.parametrize("name,li", FULL, ids=lambda v: str(v))
def test_full_size_linear(name, li):
    wl = W.WORKLOADS[name]
    lin = wl.linears[li]
    data = W.generate_linear(wl, li)
    check_linear(lin, data, wl.rowwise, sampled=True, seed=li + 1)


def test_rowwise_at_headline_shape_with_gaussian_inputs():
    """Rowwise scaling on the plain 8B FFN w1 inputs (the outlier case covers
    Student-t activations)."""
    wl = W.WORKLOADS["ffn8b_tw"]
    lin = wl.linears[0]
    data = W.generate_linear(wl, 0)
    check_linear(lin, data, True, sampled=True, seed=9)


def test_pipelined_step_equals_serial():
    """PipelinedStep (quantizes on a side stream) gives the outputs of the
    linears run in turn, also when the inputs change between steps on the
    main stream."""
    shapes = ((512, 1024, 256), (512, 1024, 256), (512, 256, 1024))

    def make(seed):
        x = G.dev_bf16(W.random_bf16(seed, (512, 256), 1.0, 0))
        ins = []
        for li, (M, N, K) in enumerate(shapes):
            xx = x if K == 256 else G.dev_bf16(W.random_bf16(seed, (M, K), 1.0, 10 + li))
            ins.append((xx, G.dev_bf16(W.random_bf16(seed, (N, K), 0.02, 20 + li)),
                        G.dev_bf16(W.random_bf16(seed, (M, N), 1e-2, 30 + li))))
        return ins
    a, b = make(71), make(72)
    steps = [ops.LinearStep(x.clone(), w.clone(), dy.clone()) for x, w, dy in a]
    pipe = ops.PipelinedStep(steps)
    got = []
    for ins in (a, b):
        for ls, (x, w, dy) in zip(steps, ins):     # new inputs, written on the main stream
            ls.x.copy_(x); ls.w.copy_(w); ls.dy.copy_(dy)
        G.say("pipelined step")
        pipe.run()
        got.append([t.clone() for ls in steps for t in (ls.out, ls.grad_x, ls.grad_w)])
    torch.cuda.synchronize()
    for ins, g in zip((a, b), got):
        ref = [ops.LinearStep(x, w, dy) for x, w, dy in ins]
        for r in ref:
            r.run()
        torch.cuda.synchronize()
        want = [t for r in ref for t in (r.out, r.grad_x, r.grad_w)]
        assert all(torch.equal(p, q) for p, q in zip(g, want))


@pytest.mark.parametrize("e5m2", [False, True], ids=["e4m3_grad", "e5m2_grad"])
@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_grouped_step_equals_serial(rowwise, e5m2):
    """GroupedStep (X of w1 and w3 quantized once, each linear's GEMMs in one
    grouped launch, w1's grad_W in w3's) gives the outputs of the three
    LinearSteps run alone; with E5M2 gradients too, where the forward GEMM
    (E4M3 X) must not be read in the gradients' format."""
    M, D, H = 528, 272, 784
    x = G.dev_bf16(W.random_bf16(73, (M, D), 1.0, 0))
    h = G.dev_bf16(W.random_bf16(73, (M, H), 1.0, 1))
    ws = [G.dev_bf16(W.random_bf16(73, s, 0.02, 2 + i))
          for i, s in enumerate(((H, D), (H, D), (D, H)))]
    dys = [G.dev_bf16(W.random_bf16(73, s, 1e-2, 5 + i))
           for i, s in enumerate(((M, H), (M, H), (M, D)))]
    s1 = ops.LinearStep(x, ws[0], dys[0], rowwise, e5m2_grad=e5m2)
    s3 = ops.LinearStep(x, ws[1], dys[1], rowwise, e5m2_grad=e5m2, qx=s1.qx)
    s2 = ops.LinearStep(h, ws[2], dys[2], rowwise, e5m2_grad=e5m2)
    grouped = ops.GroupedStep([s1, s3, s2])
    # w1: grad_x (contraction H) before fwd (D); w3 adds both grad_W
    # (contraction M); w2: fwd (H), grad_w (M), grad_x (D)
    assert grouped.plan == [[("grad_x", 0), ("fwd", 0)],
                            [("grad_x", 1), ("grad_w", 0), ("grad_w", 1), ("fwd", 1)],
                            [("fwd", 2), ("grad_w", 2), ("grad_x", 2)]]
    G.say("grouped step", (M, D, H), "rowwise", rowwise, "e5m2", e5m2)
    grouped.run()
    got = [t.clone() for ls in (s1, s3, s2) for t in (ls.out, ls.grad_x, ls.grad_w)]
    ref = [ops.LinearStep(xx, w, dy, rowwise, e5m2_grad=e5m2) for xx, w, dy in
           ((x, ws[0], dys[0]), (x, ws[1], dys[1]), (h, ws[2], dys[2]))]
    for r in ref:
        r.run()
    torch.cuda.synchronize()
    want = [t for r in ref for t in (r.out, r.grad_x, r.grad_w)]
    for i, (p, q) in enumerate(zip(got, want)):
        assert torch.equal(p, q), "output %d" % i
