"""GPU parity of the E5M2 gradient path: the device E5M2 conversion on every
fp32 input of its rounding band, quantize of dY to E5M2 (bytes and scales
bit for bit), the E5M2 x E4M3 backward GEMMs against the oracle's mixed
GEMM, and the whole linear with an E5M2 gradient at the Llama-3.1-8B FFN
shape."""
import numpy as np
import pytest
import torch

import oracle
from float8_mixed_precision_amd import ops
from float8_mixed_precision_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def test_encode_e5m2_band_exhaustive():
    """Every positive fp32 pattern of biased exponents 103..144 (from below
    half the smallest subnormal, 2^-17, to past saturation at 57344), and
    their negatives."""
    for e in range(103, 145, 2):
        G.say("encode e5m2 exponents", e, e + 1)
        bits = np.arange(e << 23, (e + 2) << 23, dtype=np.uint32)
        y = bits.view(np.float32)
        yd = torch.from_numpy(y).to(G.DEV)
        got = G.host(ops.fp8_linear_encode_e5m2(yd))
        want = oracle.e5m2_encode(y)
        assert np.array_equal(got, want), "exponent %d" % e
        got_neg = G.host(ops.fp8_linear_encode_e5m2(-yd))
        assert np.array_equal(got_neg, want ^ 0x80), "negative, exponent %d" % e


def test_encode_e5m2_random_and_special():
    rng = np.random.default_rng(51)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000,
                        1, 0x80000001, 0x7F7FFFFF, 0xFF7FFFFF, 0x47600000, 0x47700000,
                        0x37800000, 0x37000000, 0x36800000], np.uint32)
    y = np.concatenate([bits, special]).view(np.float32)
    for n in (y.size, 3, 1):
        G.say("encode e5m2 random", n)
        got = G.host(ops.fp8_linear_encode_e5m2(torch.from_numpy(y[:n].copy()).to(G.DEV)))
        want = oracle.e5m2_encode(y[:n])
        nan = np.isnan(y[:n])
        assert np.all((got[nan] & 0x7F) > 0x7C), "NaN must give a NaN code"
        assert np.array_equal(got[~nan], want[~nan])


def _quantize_e5m2(bits, rowwise):
    qz = ops.fp8_linear_quantize(G.dev_bf16(bits), rowwise, e5m2=True)
    torch.cuda.synchronize()
    return G.host(qz.q), G.host(qz.qt), G.host(qz.scale), G.host(qz.scale_t), G.host(qz.amax)


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
@pytest.mark.parametrize("shape", [(16, 16), (272, 400), (48, 4112), (1040, 80)],
                         ids=lambda s: "%dx%d" % s)
def test_quantize_e5m2(shape, rowwise):
    rng = np.random.default_rng(52)
    cases = {"grad": W.random_bf16(52, shape, 1e-2, 0),
             "student_t": W.to_bf16_bits(rng.standard_t(3, size=shape).astype(np.float32) * 1e-3),
             "tiny": W.random_bf16(52, shape, 1e-30, 1)}
    for name, x in cases.items():
        G.say("quantize e5m2", shape, name, "rowwise", rowwise)
        G.assert_quantize_equal(_quantize_e5m2(x, rowwise), oracle.quantize_e5m2(x, rowwise),
                                "%s %s" % (shape, name))


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_quantize_e5m2_empty_and_special(rowwise):
    x = torch.empty((0, 32), dtype=torch.bfloat16, device=G.DEV)
    qz = ops.fp8_linear_quantize(x, rowwise, e5m2=True)
    torch.cuda.synchronize()
    if not rowwise:
        assert G.host(qz.scale)[0] == oracle.scale_from_amax_e5m2(0.0)
    z = np.zeros((272, 400), np.uint16)
    z[5, 7] = 0x3F80
    G.assert_quantize_equal(_quantize_e5m2(z, rowwise), oracle.quantize_e5m2(z, rowwise), "single")


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
@pytest.mark.parametrize("mnk", [(272, 400, 528), (256, 256, 16), (1040, 784, 304)],
                         ids=lambda s: "%dx%dx%d" % s)
def test_bwd_e5m2(mnk, rowwise):
    """grad_X = dY . W and grad_W = dY^T . X with dY in E5M2, fully compared
    with the oracle's E5M2 x E4M3 GEMM; the fp32 grad_W rounds to the bf16
    one."""
    M, N, K = mnk
    x = W.random_bf16(53, (M, K), 1.0, 2)
    w = W.random_bf16(53, (N, K), 0.02, 3)
    dy = W.random_bf16(53, (M, N), 1e-2, 4)
    G.say("bwd e5m2", mnk, "rowwise", rowwise)
    qx = ops.fp8_linear_quantize(G.dev_bf16(x), rowwise)
    qw = ops.fp8_linear_quantize(G.dev_bf16(w), rowwise)
    qdy = ops.fp8_linear_quantize(G.dev_bf16(dy), rowwise, e5m2=True)
    gx, gw = ops.fp8_linear_bwd(qdy.q, qdy.scale, qdy.qt, qdy.scale_t, qw.qt, qw.scale_t,
                                qx.qt, qx.scale_t, M, N, K, rowwise, e5m2=True)
    g32 = ops.fp8_linear_bwd_w_f32(qdy.qt, qdy.scale_t, qx.qt, qx.scale_t, M, N, K, rowwise,
                                   e5m2=True)
    torch.cuda.synchronize()
    # the oracle's own codes (equal to the device's, checked first)
    rdy = oracle.quantize_e5m2(dy, rowwise)
    rx = oracle.quantize(x, rowwise)
    rw_ = oracle.quantize(w, rowwise)
    for name, qz, r in (("dY", qdy, rdy), ("X", qx, rx), ("W", qw, rw_)):
        G.assert_quantize_equal((G.host(qz.q), G.host(qz.qt), G.host(qz.scale),
                                 G.host(qz.scale_t), G.host(qz.amax)), r, name)
    ox = oracle.gemm_tn_mixed(rdy[0], 1, rdy[2], rw_[1], 0, rw_[3])
    G.gemm_parity(G.host(gx), ox, rdy[0], rw_[1], rdy[2], rw_[3],
                  label="e5m2 grad_x %s" % (mnk,), e5m2_a=True)
    ow = oracle.gemm_tn_mixed(rdy[1], 1, rdy[3], rx[1], 0, rx[3])
    G.gemm_parity(G.host(gw), ow, rdy[1], rx[1], rdy[3], rx[3],
                  label="e5m2 grad_w %s" % (mnk,), e5m2_a=True)
    bits = torch.from_numpy(G.host(g32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, G.host(gw))


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_linear_e5m2_full_size(rowwise):
    """Llama-3.1-8B FFN w1 with an E5M2 gradient, in the launch sequence the
    benchmark times: quantize outputs in full, GEMMs on sampled positions."""
    wl = W.WORKLOADS["ffn8b_tw"]
    lin = wl.linears[0]
    M, N, K = lin.M, lin.N, lin.K
    data = W.generate_linear(wl, 0)
    G.say("linear e5m2", (M, N, K), "rowwise", rowwise)
    step = ops.LinearStep(G.dev_bf16(data["x"]), G.dev_bf16(data["w"]), G.dev_bf16(data["dy"]),
                          rowwise, e5m2_grad=True)
    step.run()
    torch.cuda.synchronize()
    rdy = oracle.quantize_e5m2(data["dy"], rowwise)
    got = (G.host(step.qdy.q), G.host(step.qdy.qt), G.host(step.qdy.scale),
           G.host(step.qdy.scale_t), G.host(step.qdy.amax))
    G.assert_quantize_equal(got, rdy, "dY e5m2")
    rx = oracle.quantize(data["x"], rowwise)
    rw = oracle.quantize(data["w"], rowwise)
    for name, out_t, a, sa, b, sb, m_, n_ in (
            ("grad_x", step.grad_x, rdy[0], rdy[2], rw[1], rw[3], M, K),
            ("grad_w", step.grad_w, rdy[1], rdy[3], rx[1], rx[3], N, K)):
        ii, jj = G.sample_indices(m_, n_, 6000, 54)
        o = oracle.gemm_tn_mixed_sampled(a, 1, sa, b, 0, sb, ii, jj)
        G.gemm_parity(G.host(out_t)[ii, jj], o, a, b, sa, sb, ii, jj,
                      label="e5m2 full %s rowwise %s" % (name, rowwise), e5m2_a=True)
