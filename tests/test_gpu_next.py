"""GPU parity of the entry points beyond the linear's own step:

* fp8_linear_amax and fp8_linear_quantize_scaled, one GPU's share of Float8
  all-gather (shard amax, then a cast with the scale of the global amax):
  bit-exact against the oracle;
* fp8_linear_bwd_w_f32, grad_W with an fp32 output (for an fp32
  reduce-scatter): against the oracle's fp32 GEMM within the room two valid
  summation orders leave, and bit-exact against the bf16 kernel after bf16
  rounding (both epilogues read the same accumulators)."""
import numpy as np
import pytest
import torch

import oracle
from float8_mixed_precision_amd import ops
from float8_mixed_precision_amd import workloads as W
from tests import gpu_util as G
from tests import mfma_model as MM

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
SHAPES = [(16, 16), (272, 400), (48, 4112), (1040, 80), (528, 784)]


def _amax_dev(bits):
    return float(G.host(ops.fp8_linear_amax(G.dev_bf16(bits)))[0])


@pytest.mark.parametrize("shape", SHAPES + [(8192, 4096), (8192, 14336)], ids=lambda s: "%dx%d" % s)
def test_amax(shape):
    x = W.random_bf16(40, shape, 0.02 if shape[0] > 4096 else 1.0, 0)
    G.say("amax", shape)
    got = np.float32(_amax_dev(x))
    want = oracle.amax(x)
    assert got.view(np.uint32) == np.float32(want).view(np.uint32), (got, want)


def test_amax_special():
    x = W.random_bf16(41, (272, 400), 1.0, 1)
    xn = x.copy()
    xn[271, 399] = 0x7FC0                                 # NaN in the last element
    assert np.isnan(_amax_dev(xn))
    xi = x.copy()
    xi[0, 0] = 0xFF80                                     # -inf in the first
    assert np.isposinf(_amax_dev(xi))
    assert _amax_dev(np.zeros((272, 400), np.uint16)) == 0.0
    out = ops.fp8_linear_amax(torch.empty((0, 64), dtype=torch.bfloat16, device=G.DEV))
    assert float(G.host(out)[0]) == 0.0


@pytest.mark.parametrize("shape", SHAPES + [(8192, 14336)], ids=lambda s: "%dx%d" % s)
def test_quantize_scaled(shape):
    """Scales that keep, shrink and saturate the values, and the tensor's own
    scale (where the cast must equal the tensorwise quantize)."""
    x = W.random_bf16(42, shape, 1.0, 2)
    xd = G.dev_bf16(x)
    own = oracle.scale_from_amax(oracle.amax(x))
    scales = [own] if shape[0] > 4096 else [1.0, 3.7e-3, 1e5, own]
    for s in scales:
        G.say("quantize_scaled", shape, "scale", s)
        sd = torch.tensor([s], dtype=torch.float32, device=G.DEV)
        q, qt = ops.fp8_linear_quantize_scaled(xd, sd)
        torch.cuda.synchronize()
        wq, wqt = oracle.quantize_scaled(x, s)
        assert np.array_equal(G.host(q), wq), "q, scale %g" % s
        assert np.array_equal(G.host(qt), wqt), "qt, scale %g" % s


def test_all_gather_share_flow():
    """Shard amax -> (the all-reduce(max) a multi-GPU run would do across
    shards, here over two shards of one tensor on the host) -> scale -> cast
    of each shard: equals the tensorwise quantize of the whole tensor."""
    x = W.random_bf16(43, (1024, 2048), 0.02, 3)
    shards = [x[:512], x[512:]]
    amaxes = [_amax_dev(s) for s in shards]
    s = oracle.scale_from_amax(np.float32(max(amaxes)))
    sd = torch.tensor([s], dtype=torch.float32, device=G.DEV)
    qs = [ops.fp8_linear_quantize_scaled(G.dev_bf16(sh), sd)[0] for sh in shards]
    torch.cuda.synchronize()
    whole = oracle.quantize(x, False)
    assert np.array_equal(np.concatenate([G.host(q) for q in qs]), whole[0])
    assert np.float32(s).view(np.uint32) == whole[2][0].view(np.uint32)


def _f32_parity(g, o, a, b, sa, sb, ii, jj, label):
    """|G - O| <= 2 ulp_f32(O) + inv_a inv_b D (1 + 2^-20): D bounds the
    distance between the oracle's sequential fp32 accumulator and the
    instruction's (tests/mfma_model.py derives it from the reading of the
    instruction's accumulation); the two fp32 epilogue multiplies on each
    side add at most an ulp each.  Relative Frobenius <= 1e-3 as for the
    bf16 outputs."""
    g = np.asarray(g, np.float64).ravel()
    o = np.asarray(o, np.float32).ravel()
    sa = np.atleast_1d(sa).astype(np.float32)
    sb = np.atleast_1d(sb).astype(np.float32)
    inva = (np.float32(1) / sa).astype(np.float64)
    invb = (np.float32(1) / sb).astype(np.float64)
    inva = inva[ii] if inva.size > 1 else np.full(len(ii), inva[0])
    invb = invb[jj] if invb.size > 1 else np.full(len(jj), invb[0])
    dmax = MM.sum_difference_bound(a, b, ii, jj)
    ulp = np.spacing(np.abs(o)).astype(np.float64)
    allowed = 2 * ulp + inva * invb * dmax * (1 + 2.0 ** -20)
    o64 = o.astype(np.float64)
    rf = np.linalg.norm(g - o64) / max(np.linalg.norm(o64), 1e-300)
    G.say("parity f32", label, dict(n=len(g), relfro=rf,
                                     max_rel=float(np.max(np.abs(g - o64) / np.maximum(np.abs(o64), 1e-30))),
                                     max_bound_use=float(np.max(np.abs(g - o64) / allowed))))
    assert np.all(np.isfinite(g)), label
    assert rf <= 1e-3, "%s: relative Frobenius %.3g" % (label, rf)
    bad = np.abs(g - o64) > allowed
    assert not bad.any(), "%s: %d elements outside the bound" % (label, int(bad.sum()))


def _oracle_codes(x, dy, qx, qdy, rowwise):
    """The oracle's quantize of x and dy, checked equal to the device's."""
    rx = oracle.quantize(x, rowwise)
    rdy = oracle.quantize(dy, rowwise)
    for name, qz, r in (("X", qx, rx), ("dY", qdy, rdy)):
        G.assert_quantize_equal((G.host(qz.q), G.host(qz.qt), G.host(qz.scale),
                                 G.host(qz.scale_t), G.host(qz.amax)), r, name)
    return rx, rdy


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
@pytest.mark.parametrize("mnk", [(272, 400, 528), (256, 256, 16), (1040, 784, 304)],
                         ids=lambda s: "%dx%dx%d" % s)
def test_bwd_w_f32(mnk, rowwise):
    """grad_W [N, K] from dYTq [N, M] and XTq [K, M]; full comparison."""
    M, N, K = mnk
    x = W.random_bf16(44, (M, K), 1.0, 4)
    dy = W.random_bf16(44, (M, N), 1e-2, 5)
    G.say("bwd_w_f32", mnk, "rowwise", rowwise)
    qx = ops.fp8_linear_quantize(G.dev_bf16(x), rowwise)
    qdy = ops.fp8_linear_quantize(G.dev_bf16(dy), rowwise)
    g32 = ops.fp8_linear_bwd_w_f32(qdy.qt, qdy.scale_t, qx.qt, qx.scale_t, M, N, K, rowwise)
    _, g16 = ops.fp8_linear_bwd(None, None, qdy.qt, qdy.scale_t, None, None, qx.qt, qx.scale_t,
                                M, N, K, rowwise, want_x=False)
    torch.cuda.synchronize()
    rx, rdy = _oracle_codes(x, dy, qx, qdy, rowwise)
    a, sa, b, sb = rdy[1], rdy[3], rx[1], rx[3]
    o = oracle.gemm_tn_f32(a, sa, b, sb)
    ii, jj = np.divmod(np.arange(N * K), K)
    gh = G.host(g32)
    _f32_parity(gh, o, a, b, sa, sb, ii, jj, "bwd_w_f32 %s" % (mnk,))
    # the bf16 kernel rounds the same fp32 values
    bits = torch.from_numpy(gh.reshape(N, K)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(bits.view(np.uint16), G.host(g16).view(np.uint16))


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_bwd_w_f32_empty_contraction(rowwise):
    """M = 0 tokens: grad_W is the product over an empty contraction, all
    zeros (fp32 +0), whatever the output held before."""
    M, N, K = 0, 48, 80
    G.say("bwd_w_f32 empty contraction", (M, N, K), "rowwise", rowwise)
    qx = ops.fp8_linear_quantize(G.dev_bf16(np.zeros((M, K), np.uint16)), rowwise)
    qdy = ops.fp8_linear_quantize(G.dev_bf16(np.zeros((M, N), np.uint16)), rowwise)
    g32 = torch.full((N, K), -3.5, dtype=torch.float32, device=G.DEV)
    ops.fp8_linear_bwd_w_f32(qdy.qt, qdy.scale_t, qx.qt, qx.scale_t, M, N, K, rowwise, g32)
    torch.cuda.synchronize()
    assert np.array_equal(G.host(g32).view(np.uint32), np.zeros((N, K), np.uint32))


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_bwd_w_f32_full_size(rowwise):
    """The Llama-3.1-8B FFN w1 grad_W (N 14336, K 4096, contraction 8192),
    sampled against the oracle."""
    wl = W.WORKLOADS["ffn8b_tw"]
    lin = wl.linears[0]
    M, N, K = lin.M, lin.N, lin.K
    data = W.generate_linear(wl, 0)
    G.say("bwd_w_f32 full", (M, N, K), "rowwise", rowwise)
    qx = ops.fp8_linear_quantize(G.dev_bf16(data["x"]), rowwise)
    qdy = ops.fp8_linear_quantize(G.dev_bf16(data["dy"]), rowwise)
    g32 = ops.fp8_linear_bwd_w_f32(qdy.qt, qdy.scale_t, qx.qt, qx.scale_t, M, N, K, rowwise)
    _, g16 = ops.fp8_linear_bwd(None, None, qdy.qt, qdy.scale_t, None, None, qx.qt, qx.scale_t,
                                M, N, K, rowwise, want_x=False)
    torch.cuda.synchronize()
    gh = G.host(g32)
    bits = torch.from_numpy(gh).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, G.host(g16).view(np.uint16))
    rx, rdy = _oracle_codes(data["x"], data["dy"], qx, qdy, rowwise)
    a, sa, b, sb = rdy[1], rdy[3], rx[1], rx[3]
    ii, jj = G.sample_indices(N, K, 6000, 45)
    o = oracle.gemm_tn_f32_sampled(a, sa, b, sb, ii, jj)
    _f32_parity(gh[ii, jj], o, a, b, sa, sb, ii, jj, "bwd_w_f32 full rowwise %s" % rowwise)
