"""GPU parity of the three scaled fp8 GEMMs (fwd, grad_X, grad_W) against the
oracle on the same fp8 bytes: relative Frobenius <= 1e-3 and every element
within 2 bf16 ulps plus the room two fp32 summation orders may differ by."""
import numpy as np
import pytest
import torch

import oracle
from float8_mixed_precision_amd import ops
from float8_mixed_precision_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def run_gemm(a, sa, b, sb, rowwise):
    out = ops.fp8_linear_fwd(G.dev_u8(a), G.dev_f32(sa), G.dev_u8(b), G.dev_f32(sb), rowwise)
    torch.cuda.synchronize()
    return G.host(out)


def random_operands(m, n, k, rowwise, seed):
    """fp8 operands as quantize produces them from Gaussian bf16 data."""
    xa = W.random_bf16(seed, (m, k), 1.0, 0)
    xb = W.random_bf16(seed, (n, k), 0.02, 1)
    a, _, sa, _, _ = oracle.quantize(xa, rowwise)
    b, _, sb, _, _ = oracle.quantize(xb, rowwise)
    return a, sa, b, sb


SHAPES = [(16, 16, 16), (256, 256, 128), (272, 400, 208), (528, 784, 336),
          (48, 1040, 4112), (1040, 48, 272), (512, 512, 1024)]


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_gemm_full_compare(shape, rowwise):
    """Every output, on shapes that span several 256x256 tiles and leave
    ragged M, N and K tails (multiples of 16 only)."""
    m, n, k = shape
    a, sa, b, sb = random_operands(m, n, k, rowwise, seed=sum(shape))
    G.say("gemm", shape, "rowwise", rowwise)
    got = run_gemm(a, sa, b, sb, rowwise)
    want = oracle.gemm_tn(a, sa, b, sb)
    G.gemm_parity(got, want, a, b, sa, sb, label="gemm %s rw=%s" % (shape, rowwise))


def test_gemm_extreme_codes():
    """All-448 operands (largest products, long sums), all-smallest-subnormal
    operands, and alternating signs (exact cancellation)."""
    m, n, k = 272, 272, 2064
    cases = {
        "max": (np.full((m, k), 0x7E, np.uint8), np.full((n, k), 0x7E, np.uint8)),
        "min_sub": (np.full((m, k), 0x01, np.uint8), np.full((n, k), 0x81, np.uint8)),
        "cancel": (np.tile(np.array([0x7E, 0xFE], np.uint8), (m, k // 2)),
                   np.full((n, k), 0x40, np.uint8)),
    }
    for name, (a, b) in cases.items():
        for sa, sb in ((1.0, 1.0), (448.0, 3.0e-2)):
            G.say("gemm extreme", name, sa, sb)
            got = run_gemm(a, np.float32(sa), b, np.float32(sb), False)
            want = oracle.gemm_tn(a, np.float32(sa), b, np.float32(sb))
            G.gemm_parity(got, want, a, b, np.float32(sa), np.float32(sb), label=name)


def test_gemm_k_zero_and_empty():
    G.say("gemm K=0 / M=0")
    a = torch.empty((32, 0), dtype=torch.uint8, device=G.DEV)
    b = torch.empty((48, 0), dtype=torch.uint8, device=G.DEV)
    s = G.dev_f32(np.float32(2.0))
    out = torch.full((32, 48), 7.0, dtype=torch.bfloat16, device=G.DEV)
    ops.fp8_linear_fwd(a, s, b, s, False, out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    # M = 0: nothing to write, must succeed
    a0 = torch.empty((0, 64), dtype=torch.uint8, device=G.DEV)
    b0 = torch.zeros((48, 64), dtype=torch.uint8, device=G.DEV)
    o0 = torch.empty((0, 48), dtype=torch.bfloat16, device=G.DEV)
    ops.fp8_linear_fwd(a0, s, b0, s, False, o0)
    torch.cuda.synchronize()


def test_gemm_tensorwise_equals_constant_rowwise():
    m, n, k = 272, 400, 208
    a, sa, b, sb = random_operands(m, n, k, False, seed=3)
    G.say("gemm tensorwise vs constant rowwise")
    t = run_gemm(a, sa, b, sb, False)
    r = run_gemm(a, np.full(m, sa[0], np.float32), b, np.full(n, sb[0], np.float32), True)
    assert np.array_equal(t, r)


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_linear_step_mid_size(rowwise):
    """One linear through LinearStep (the launch sequence the benchmark times)
    on a ragged mid-size shape: quantize outputs bit-exact, all three GEMMs
    in tolerance, every output compared."""
    M, N, K = 528, 784, 336
    x = W.random_bf16(11, (M, K), 1.0, 0)
    w = W.random_bf16(11, (N, K), 0.02, 1)
    dy = W.random_bf16(11, (M, N), 1e-2, 2)
    step = ops.LinearStep(G.dev_bf16(x), G.dev_bf16(w), G.dev_bf16(dy), rowwise)
    G.say("linear step mid", (M, N, K), "rowwise", rowwise)
    step.run()
    torch.cuda.synchronize()
    ox, ow, ody = (oracle.quantize(t, rowwise) for t in (x, w, dy))
    for name, qz, ref in (("X", step.qx, ox), ("W", step.qw, ow), ("dY", step.qdy, ody)):
        got = (G.host(qz.q), G.host(qz.qt), G.host(qz.scale), G.host(qz.scale_t), G.host(qz.amax))
        G.assert_quantize_equal(got, ref, "quantize " + name)
    out = oracle.gemm_tn(ox[0], ox[2], ow[0], ow[2])
    G.gemm_parity(G.host(step.out), out, ox[0], ow[0], ox[2], ow[2], label="fwd")
    gx = oracle.gemm_tn(ody[0], ody[2], ow[1], ow[3])
    G.gemm_parity(G.host(step.grad_x), gx, ody[0], ow[1], ody[2], ow[3], label="grad_x")
    gw = oracle.gemm_tn(ody[1], ody[3], ox[1], ox[3])
    G.gemm_parity(G.host(step.grad_w), gw, ody[1], ox[1], ody[3], ox[3], label="grad_w")


@pytest.mark.parametrize("e5m2", [False, True], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_gemm_grouped(rowwise, e5m2):
    """Up to four GEMMs of different shapes (ragged, one empty, one with a K
    tail) in one launch: each output equals its own launch bit for bit, and
    the first is checked against the oracle."""
    shapes = [(272, 400, 208), (0, 64, 128), (528, 784, 336), (256, 256, 16)]
    ops_in, outs = [], []
    for i, (m, n, k) in enumerate(shapes):
        xa = W.random_bf16(80 + i, (max(m, 16), k), 1e-2 if e5m2 else 1.0, 0)[:m]
        xb = W.random_bf16(80 + i, (n, k), 0.02, 1)
        qa = (oracle.quantize_e5m2 if e5m2 else oracle.quantize)(xa, rowwise)
        qb = oracle.quantize(xb, rowwise)
        ops_in.append((qa[0], qa[2], qb[0], qb[2]))
        outs.append(torch.full((m, n), 3.0, dtype=torch.bfloat16, device=G.DEV))
    dev = [(G.dev_u8(a), G.dev_f32(sa), G.dev_u8(b), G.dev_f32(sb)) for a, sa, b, sb in ops_in]
    G.say("gemm grouped", shapes, "rowwise", rowwise, "e5m2", e5m2)
    ops.fp8_linear_gemm_grouped([d + (o,) for d, o in zip(dev, outs)], rowwise, e5m2=e5m2)
    single = []
    for (a, sa, b, sb), (m, n, k) in zip(dev, shapes):
        o = torch.full((m, n), 5.0, dtype=torch.bfloat16, device=G.DEV)
        ops.fp8_linear_gemm_grouped([(a, sa, b, sb, o)], rowwise, e5m2=e5m2)
        single.append(o)
    torch.cuda.synchronize()
    for i, (g, s) in enumerate(zip(outs, single)):
        assert torch.equal(g, s), "problem %d differs from its own launch" % i
    a, sa, b, sb = ops_in[0]
    want = oracle.gemm_tn_mixed(a, 1 if e5m2 else 0, sa, b, 0, sb)
    G.gemm_parity(G.host(outs[0]), want, a, b, sa, sb, label="grouped[0]", e5m2_a=e5m2)
    # a single problem through the group entry equals fp8_linear_fwd
    if not e5m2:
        f = ops.fp8_linear_fwd(dev[2][0], dev[2][1], dev[2][2], dev[2][3], rowwise)
        torch.cuda.synchronize()
        assert torch.equal(f, single[2])


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_gemm_grouped_mixed_k(rowwise):
    """A grouped launch whose problems have different K, the first with K = 0
    (an all-zero output) and the rest given in increasing K: every output
    equals its own launch bit for bit, and the longest is checked against
    the oracle."""
    shapes = [(96, 80, 0), (272, 400, 208), (304, 256, 1024), (528, 272, 2048)]
    ops_in, outs = [], []
    for i, (m, n, k) in enumerate(shapes):
        if k == 0:
            qa = (np.zeros((m, 0), np.uint8), np.ones(m if rowwise else 1, np.float32))
            qb = (np.zeros((n, 0), np.uint8), np.ones(n if rowwise else 1, np.float32))
            ops_in.append((qa[0], qa[1], qb[0], qb[1]))
        else:
            qa = oracle.quantize(W.random_bf16(90 + i, (m, k), 1.0, 0), rowwise)
            qb = oracle.quantize(W.random_bf16(90 + i, (n, k), 0.02, 1), rowwise)
            ops_in.append((qa[0], qa[2], qb[0], qb[2]))
        outs.append(torch.full((m, n), 3.0, dtype=torch.bfloat16, device=G.DEV))
    dev = [(G.dev_u8(a), G.dev_f32(sa), G.dev_u8(b), G.dev_f32(sb)) for a, sa, b, sb in ops_in]
    G.say("gemm grouped mixed K", shapes, "rowwise", rowwise)
    ops.fp8_linear_gemm_grouped([d + (o,) for d, o in zip(dev, outs)], rowwise)
    single = []
    for (a, sa, b, sb), (m, n, k) in zip(dev, shapes):
        o = torch.full((m, n), 5.0, dtype=torch.bfloat16, device=G.DEV)
        ops.fp8_linear_gemm_grouped([(a, sa, b, sb, o)], rowwise)
        single.append(o)
    torch.cuda.synchronize()
    assert torch.all(outs[0] == 0)
    for i, (g, s1) in enumerate(zip(outs, single)):
        assert torch.equal(g, s1), "problem %d differs from its own launch" % i
    a, sa, b, sb = ops_in[3]
    want = oracle.gemm_tn(a, sa, b, sb)
    G.gemm_parity(G.host(outs[3]), want, a, b, sa, sb, label="mixed K [3]")


def _sampled_parity_at(a, sa, b, sb, out, rows, cols, label):
    """The oracle's values at rows x cols (every pair) against out's."""
    ii, jj = (np.repeat(rows, len(cols)), np.tile(cols, len(rows)))
    want = oracle.gemm_tn_sampled(a, sa, b, sb, ii, jj)
    got = G.host(out[torch.as_tensor(ii, device=G.DEV), torch.as_tensor(jj, device=G.DEV)])
    G.gemm_parity(got, want, a, b, sa, sb, ii=ii, jj=jj, label=label)


def test_gemm_output_at_the_offset_limit():
    """The largest accepted bf16 output: [32752, 32768] is 2^31 - 2^20 bytes,
    so the kernel's 32-bit store offsets reach their largest values.  The
    first and last rows and columns and a random sample match the oracle,
    and a guard region right after the output stays untouched."""
    M, N, K = 32752, 32768, 256
    rng = np.random.default_rng(93)
    import tests.pins as pins
    a, b = pins.random_codes(rng, (M, K)), pins.random_codes(rng, (N, K))
    sa, sb = np.float32(3.5), np.float32(0.75)
    guard = 1 << 16
    buf = torch.full((M * N + guard,), -7.0, dtype=torch.bfloat16, device=G.DEV)
    out = buf[:M * N].view(M, N)
    G.say("gemm at the output offset limit", (M, N, K))
    ops.fp8_linear_fwd(G.dev_u8(a), G.dev_f32(sa), G.dev_u8(b), G.dev_f32(sb), False, out=out)
    torch.cuda.synchronize()
    assert bool(torch.all(buf[M * N:] == -7.0)), "write past the output"
    rows = np.unique(np.concatenate([[0, 1, M - 2, M - 1], rng.integers(0, M, 24)]))
    cols = np.unique(np.concatenate([[0, 1, N - 2, N - 1], rng.integers(0, N, 24)]))
    _sampled_parity_at(a, sa, b, sb, out, rows, cols, "output offset limit")


def test_gemm_operand_at_the_offset_limit():
    """The largest accepted fp8 operand: A [65520, 32768] is 2^31 - 2^19
    bytes, so the kernel's 32-bit load offsets reach their largest values
    (N = 16: one partial tile column)."""
    M, N, K = 65520, 16, 32768
    rng = np.random.default_rng(94)

    def codes(shape):          # random finite E4M3 codes, generated as bytes
        c = rng.integers(0, 256, size=shape, dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] ^= 1
        return c

    a, b = codes((M, K)), codes((N, K))
    sa, sb = np.float32(1.25), np.float32(2.0)
    G.say("gemm at the operand offset limit", (M, N, K))
    out = ops.fp8_linear_fwd(G.dev_u8(a), G.dev_f32(sa), G.dev_u8(b), G.dev_f32(sb), False)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, M - 2, M - 1], rng.integers(0, M, 60)]))
    _sampled_parity_at(a, sa, b, sb, out, rows, np.arange(N), "operand offset limit")
