"""GPU parity of the SwiGLU feed-forward block's own pieces:

* fp8_swiglu_fwd: h = silu(a) * b bit for bit against the oracle (every bf16
  pattern of a, special values, ragged shapes, the Llama-3.1-8B FFN size),
  and the quantize of h that follows it (codes, scales, amax) bit for bit
  against the oracle's quantize of the oracle's h;
* fp8_swiglu_bwd: da, db and their quantizes (E4M3 and E5M2) likewise;
* fp8_linear_bwd_x_acc: the GEMM added into an existing bf16 grad_x, against
  the oracle's GEMM then bf16 sum within the summation-order room, and bit
  for bit against torch's bf16 addition of the plain GEMM's output;
* the whole block (SwiGLUFFNStep) against the oracle's chain of the same
  steps, with distinct input scales so that a swapped operand, scale or
  transpose shows as an O(1) error.

Every oracle input is the seeded synthetic data or an oracle output."""
import numpy as np
import pytest
import torch

import oracle
from float8_mixed_precision_amd import ops
from float8_mixed_precision_amd import workloads as W
from tests import gpu_util as G
from tests import mfma_model as MM

pytestmark = pytest.mark.gpu

SHAPES = [(16, 16), (272, 400), (48, 4112), (1040, 80), (528, 784)]
RW_IDS = ["tensorwise", "rowwise"]


def _value(bits):
    return oracle.bf16_to_f32(bits)


def assert_bf16_equal(got, want, label):
    """Bit-equal, except that any NaN matches any NaN."""
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    assert got.shape == want.shape, (label, got.shape, want.shape)
    gn = np.isnan(_value(got))
    wn = np.isnan(_value(want))
    assert np.array_equal(gn, wn), "%s: NaN positions differ" % label
    bad = (got != want) & ~wn
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d elements differ, first %s: gpu %#x oracle %#x"
                             % (label, int(bad.sum()), i, int(got[i]), int(want[i])))


def _host_q(qz):
    return G.host(qz.q), G.host(qz.qt), G.host(qz.scale), G.host(qz.scale_t), G.host(qz.amax)


def _inputs(shape, seed):
    a = W.random_bf16(seed, shape, 3.0, 0)
    b = W.random_bf16(seed, shape, 1.0, 1)
    dh = W.random_bf16(seed, shape, 1e-2, 2)
    return a, b, dh


def _run_fwd(a, b, rowwise):
    h, qh = ops.fp8_swiglu_fwd(G.dev_bf16(a), G.dev_bf16(b), rowwise)
    torch.cuda.synchronize()
    return G.host(h), _host_q(qh)


def _run_bwd(dh, a, b, rowwise, e5m2):
    da, db, qa, qb = ops.fp8_swiglu_bwd(G.dev_bf16(dh), G.dev_bf16(a), G.dev_bf16(b), rowwise,
                                        e5m2=e5m2)
    torch.cuda.synchronize()
    return G.host(da), G.host(db), _host_q(qa), _host_q(qb)


@pytest.mark.parametrize("rowwise", [False, True], ids=RW_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%d" % s)
def test_swiglu_fwd(shape, rowwise):
    a, b, _ = _inputs(shape, 60)
    G.say("swiglu fwd", shape, "rowwise", rowwise)
    h, q = _run_fwd(a, b, rowwise)
    want_h = oracle.swiglu_fwd(a, b)
    assert_bf16_equal(h, want_h, "h %s" % (shape,))
    G.assert_quantize_equal(q, oracle.quantize(want_h, rowwise), "quantize of h %s" % (shape,))


def test_swiglu_fwd_every_bf16_gate():
    """a takes every bf16 pattern (NaNs, infinities, subnormals included, and
    both sides of the range whose silu values come from the table) against
    b = 1 and against random b."""
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(4096, 16)
    for name, b in (("b=1", np.full(a.shape, 0x3F80, np.uint16)),
                    ("b random", W.random_bf16(61, a.shape, 1.0, 0))):
        G.say("swiglu fwd every gate", name)
        h, _ = _run_fwd(a, b, False)
        assert_bf16_equal(h, oracle.swiglu_fwd(a, b), name)


@pytest.mark.parametrize("rowwise", [False, True], ids=RW_IDS)
def test_swiglu_bwd_every_bf16_gate(rowwise):
    """da and db with a taking every bf16 pattern (both sides of the range
    whose silu values come from the table, zeros, subnormals, infinities,
    NaN), random b and dh."""
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(4096, 16)
    b = W.random_bf16(68, a.shape, 1.0, 0)
    dh = W.random_bf16(68, a.shape, 1e-2, 1)
    G.say("swiglu bwd every gate", "rowwise", rowwise)
    da, db, _, _ = _run_bwd(dh, a, b, rowwise, False)
    wda, wdb = oracle.swiglu_bwd(dh, a, b)
    assert_bf16_equal(da, wda, "da every gate")
    assert_bf16_equal(db, wdb, "db every gate")


@pytest.mark.parametrize("rowwise", [False, True], ids=RW_IDS)
def test_swiglu_special_and_empty(rowwise):
    a, b, dh = _inputs((272, 400), 62)
    a[0, :6] = [0x7FC0, 0xFF80, 0x7F80, 0x0001, 0x8000, 0xC4FA]   # NaN -inf inf sub -0 -2000
    a[271, 399] = 0x7F7F                                         # largest finite
    b[5, 5] = 0x7F80
    G.say("swiglu special", "rowwise", rowwise)
    h, q = _run_fwd(a, b, rowwise)
    want_h = oracle.swiglu_fwd(a, b)
    assert_bf16_equal(h, want_h, "h special")
    am = G.host(ops.fp8_swiglu_fwd(G.dev_bf16(a), G.dev_bf16(b), rowwise)[1].amax)
    assert np.isnan(am[0]), "a NaN in h must make its amax NaN"
    da, db, _, _ = _run_bwd(dh, a, b, rowwise, False)
    wda, wdb = oracle.swiglu_bwd(dh, a, b)
    assert_bf16_equal(da, wda, "da special")
    assert_bf16_equal(db, wdb, "db special")
    e = torch.empty((0, 64), dtype=torch.bfloat16, device=G.DEV)
    h0, q0 = ops.fp8_swiglu_fwd(e, e, rowwise)
    torch.cuda.synchronize()
    if not rowwise:
        assert G.host(q0.scale)[0] == oracle.scale_from_amax(0.0)
    _, _, qa0, qb0 = ops.fp8_swiglu_bwd(e, e, e, rowwise, e5m2=True)
    torch.cuda.synchronize()
    if not rowwise:
        assert G.host(qb0.scale)[0] == oracle.scale_from_amax_e5m2(0.0)


@pytest.mark.parametrize("e5m2", [False, True], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("rowwise", [False, True], ids=RW_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%d" % s)
def test_swiglu_bwd(shape, rowwise, e5m2):
    a, b, dh = _inputs(shape, 63)
    G.say("swiglu bwd", shape, "rowwise", rowwise, "e5m2", e5m2)
    da, db, qa, qb = _run_bwd(dh, a, b, rowwise, e5m2)
    wda, wdb = oracle.swiglu_bwd(dh, a, b)
    assert_bf16_equal(da, wda, "da %s" % (shape,))
    assert_bf16_equal(db, wdb, "db %s" % (shape,))
    quant = oracle.quantize_e5m2 if e5m2 else oracle.quantize
    G.assert_quantize_equal(qa, quant(wda, rowwise), "quantize of da %s" % (shape,))
    G.assert_quantize_equal(qb, quant(wdb, rowwise), "quantize of db %s" % (shape,))


def test_swiglu_workspace_reuse():
    """A workspace holding stale maxima from an earlier, larger call."""
    a, b, dh = _inputs((528, 784), 64)
    ws = ops.alloc_swiglu_workspace(528, 784, False, G.DEV)
    ws.fill_(0x7F)
    small = (a[:272, :400].copy(), b[:272, :400].copy(), dh[:272, :400].copy())
    G.say("swiglu workspace reuse")
    h, qh = ops.fp8_swiglu_fwd(G.dev_bf16(small[0]), G.dev_bf16(small[1]), False, workspace=ws)
    _, _, qa, qb = ops.fp8_swiglu_bwd(*[G.dev_bf16(t) for t in (small[2], small[0], small[1])],
                                      False, workspace=ws)
    torch.cuda.synchronize()
    want_h = oracle.swiglu_fwd(small[0], small[1])
    G.assert_quantize_equal(_host_q(qh), oracle.quantize(want_h, False), "h after stale ws")
    wda, wdb = oracle.swiglu_bwd(small[2], small[0], small[1])
    G.assert_quantize_equal(_host_q(qa), oracle.quantize(wda, False), "da after stale ws")
    G.assert_quantize_equal(_host_q(qb), oracle.quantize(wdb, False), "db after stale ws")


@pytest.mark.parametrize("rowwise", [False, True], ids=RW_IDS)
def test_swiglu_full_size(rowwise):
    """The Llama-3.1-8B FFN hidden activation, [8192, 14336]: h, da, db and
    all three quantizes in full, in the launch sequence the block uses."""
    shape = (8192, 14336)
    a = W.random_bf16(65, shape, 3.0, 0)
    b = W.random_bf16(65, shape, 1.0, 1)
    G.say("swiglu fwd full", shape, "rowwise", rowwise)
    h, q = _run_fwd(a, b, rowwise)
    want_h = oracle.swiglu_fwd(a, b)
    assert_bf16_equal(h, want_h, "h full")
    G.assert_quantize_equal(q, oracle.quantize(want_h, rowwise), "quantize of h full")
    del h, q, want_h
    dh = W.random_bf16(65, shape, 1e-2, 2)
    G.say("swiglu bwd full", shape, "rowwise", rowwise)
    da, db, qa, qb = _run_bwd(dh, a, b, rowwise, True)
    wda, wdb = oracle.swiglu_bwd(dh, a, b)
    assert_bf16_equal(da, wda, "da full")
    assert_bf16_equal(db, wdb, "db full")
    G.assert_quantize_equal(qa, oracle.quantize_e5m2(wda, rowwise), "quantize of da full")
    G.assert_quantize_equal(qb, oracle.quantize_e5m2(wdb, rowwise), "quantize of db full")


# ------------------------------------------------------- accumulate GEMM --

def _acc_parity(got, g_orc, r_orc, a, b, sa, sb, ii, jj, e5m2_a, label):
    """|G - R| <= 2 ulp(g) + 2 ulp(R) + inv_a inv_b D (1 + 2^-20): the room
    between the oracle's and the instruction's accumulators (D, derived in
    tests/mfma_model.py), the bf16 rounding of the GEMM result, and the
    rounding of the sum."""
    g = _value(np.asarray(got, np.uint16).ravel()).astype(np.float64)
    r = _value(np.asarray(r_orc, np.uint16).ravel()).astype(np.float64)
    go = np.asarray(g_orc, np.uint16).ravel()
    ro = np.asarray(r_orc, np.uint16).ravel()
    ulp = lambda o: np.abs(_value((o & 0x7FFF) + 1).astype(np.float64) - np.abs(_value(o)))
    sa = np.atleast_1d(sa).astype(np.float32)
    sb = np.atleast_1d(sb).astype(np.float32)
    inva = (np.float32(1) / sa).astype(np.float64)
    invb = (np.float32(1) / sb).astype(np.float64)
    inva = inva[ii] if inva.size > 1 else np.full(len(ii), inva[0])
    invb = invb[jj] if invb.size > 1 else np.full(len(jj), invb[0])
    dmax = MM.sum_difference_bound(a, b, ii, jj, e5m2_a)
    allowed = 2 * ulp(go) + 2 * ulp(ro) + inva * invb * dmax * (1 + 2.0 ** -20)
    rf = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    G.say("parity acc", label, dict(n=len(g), relfro=rf))
    assert np.all(np.isfinite(g)), label
    assert rf <= 1e-3, "%s: relative Frobenius %.3g" % (label, rf)
    bad = np.abs(g - r) > allowed
    assert not bad.any(), "%s: %d elements outside the bound" % (label, int(bad.sum()))


@pytest.mark.parametrize("e5m2", [False, True], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("rowwise", [False, True], ids=RW_IDS)
@pytest.mark.parametrize("mnk", [(272, 400, 528), (256, 256, 16), (1040, 784, 304)],
                         ids=lambda s: "%dx%dx%d" % s)
def test_bwd_x_acc(mnk, rowwise, e5m2):
    M, N, K = mnk
    dy = W.random_bf16(66, (M, N), 1e-2, 0)
    w = W.random_bf16(66, (N, K), 0.02, 1)
    c = W.random_bf16(66, (M, K), 1e-3, 2)          # the first contribution
    rdy = (oracle.quantize_e5m2 if e5m2 else oracle.quantize)(dy, rowwise)
    rw_ = oracle.quantize(w, rowwise)
    G.say("bwd_x_acc", mnk, "rowwise", rowwise, "e5m2", e5m2)
    qdy = ops.fp8_linear_quantize(G.dev_bf16(dy), rowwise, e5m2=e5m2)
    qw = ops.fp8_linear_quantize(G.dev_bf16(w), rowwise)
    gx = G.dev_bf16(c)
    ops.fp8_linear_bwd_x_acc(qdy.q, qdy.scale, qw.qt, qw.scale_t, M, N, K, gx, rowwise,
                             e5m2=e5m2)
    plain, _ = ops.fp8_linear_bwd(qdy.q, qdy.scale, None, None, qw.qt, qw.scale_t, None, None,
                                  M, N, K, rowwise, want_w=False, e5m2=e5m2)
    torch.cuda.synchronize()
    G.assert_quantize_equal(_host_q(qdy), rdy, "dY codes")
    G.assert_quantize_equal(_host_q(qw), rw_, "W codes")
    got = G.host(gx)
    # the epilogue's sum is torch's bf16 addition of the plain GEMM's output
    tsum = (torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).to(G.DEV) + plain)
    assert np.array_equal(got, G.host(tsum)), "accumulate differs from bf16 add of the GEMM"
    g_orc = oracle.gemm_tn_mixed(rdy[0], 1 if e5m2 else 0, rdy[2], rw_[1], 0, rw_[3])
    r_orc = oracle.add_bf16(g_orc, c)
    ii, jj = np.divmod(np.arange(M * K), K)
    _acc_parity(got, g_orc, r_orc, rdy[0], rw_[1], rdy[2], rw_[3], ii, jj, e5m2,
                "acc %s" % (mnk,))


@pytest.mark.parametrize("rowwise", [False, True], ids=RW_IDS)
def test_bwd_x_acc_empty_contraction(rowwise):
    """N = 0: the product over an empty contraction is zero, so grad_x
    becomes the bf16 sum of itself and a zero product (the oracle's bf16
    addition): unchanged, except that -0 turns into +0."""
    M, N, K = 64, 0, 48
    c = W.random_bf16(67, (M, K), 1e-3, 2)
    c.reshape(-1)[::7] = 0x8000                     # some -0 entries
    G.say("bwd_x_acc empty contraction", (M, N, K), "rowwise", rowwise)
    qdy = ops.fp8_linear_quantize(G.dev_bf16(np.zeros((M, N), np.uint16)), rowwise)
    qw = ops.fp8_linear_quantize(G.dev_bf16(np.zeros((N, K), np.uint16)), rowwise)
    gx = G.dev_bf16(c)
    ops.fp8_linear_bwd_x_acc(qdy.q, qdy.scale, qw.qt, qw.scale_t, M, N, K, gx, rowwise)
    torch.cuda.synchronize()
    want = oracle.add_bf16(np.zeros((M, K), np.uint16), c)
    assert np.array_equal(G.host(gx), want)
    assert not np.array_equal(want, c)              # the -0 entries did change


# ------------------------------------------------------------ whole block --

def _oracle_block(x, w1, w3, w2, dy, rowwise, e5m2):
    """The block's steps composed from the oracle's functions."""
    qg = oracle.quantize_e5m2 if e5m2 else oracle.quantize
    fa = 1 if e5m2 else 0
    qx, q1, q3, q2 = (oracle.quantize(t, rowwise) for t in (x, w1, w3, w2))
    a = oracle.gemm_tn(qx[0], qx[2], q1[0], q1[2])
    b = oracle.gemm_tn(qx[0], qx[2], q3[0], q3[2])
    h = oracle.swiglu_fwd(a, b)
    qh = oracle.quantize(h, rowwise)
    out = oracle.gemm_tn(qh[0], qh[2], q2[0], q2[2])
    qdy = qg(dy, rowwise)
    dh = oracle.gemm_tn_mixed(qdy[0], fa, qdy[2], q2[1], 0, q2[3])
    gw2 = oracle.gemm_tn_mixed(qdy[1], fa, qdy[3], qh[1], 0, qh[3])
    da, db = oracle.swiglu_bwd(dh, a, b)
    qda, qdb = qg(da, rowwise), qg(db, rowwise)
    gx = oracle.add_bf16(oracle.gemm_tn_mixed(qda[0], fa, qda[2], q1[1], 0, q1[3]),
                         oracle.gemm_tn_mixed(qdb[0], fa, qdb[2], q3[1], 0, q3[3]))
    gw1 = oracle.gemm_tn_mixed(qda[1], fa, qda[3], qx[1], 0, qx[3])
    gw3 = oracle.gemm_tn_mixed(qdb[1], fa, qdb[3], qx[1], 0, qx[3])
    return dict(a=a, b=b, h=h, out=out, dh=dh, grad_w2=gw2, da=da, db=db, grad_x=gx,
                grad_w1=gw1, grad_w3=gw3, qx=qx, q1=q1, q3=q3, q2=q2)


@pytest.mark.parametrize("e5m2", [False, True], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("rowwise", [False, True], ids=RW_IDS)
def test_ffn_block(rowwise, e5m2):
    """SwiGLUFFNStep (M 272, D 400, H 528) against the oracle's chain: the
    quantizes of the inputs bit for bit, a and b within the GEMM bound on
    identical codes, every later tensor within relative Frobenius 1e-2 (the
    chains then run on inputs that can differ by the GEMMs' last-bit
    rounding; a wiring error is O(1) here, as w1, w3, w2 and x have distinct
    scales)."""
    M, D, H = 272, 400, 528
    x = W.random_bf16(67, (M, D), 1.0, 0)
    w1 = W.random_bf16(67, (H, D), 0.02, 1)
    w3 = W.random_bf16(67, (H, D), 0.05, 2)
    w2 = W.random_bf16(67, (D, H), 0.01, 3)
    dy = W.random_bf16(67, (M, D), 1e-2, 4)
    G.say("ffn block", (M, D, H), "rowwise", rowwise, "e5m2", e5m2)
    blk = ops.SwiGLUFFNStep(*[G.dev_bf16(t) for t in (x, w1, w3, w2, dy)], rowwise=rowwise,
                            e5m2_grad=e5m2)
    blk.run()
    torch.cuda.synchronize()
    names = ("a", "b", "h", "out", "dh", "grad_w2", "da", "db", "grad_x", "grad_w1", "grad_w3")
    single = {n: G.host(getattr(blk, n)) for n in names}
    # a second step over the same buffers, with the independent quantizes on
    # a side stream, gives the same result
    blk.run(torch.cuda.Stream(device=G.DEV))
    torch.cuda.synchronize()
    for n in names:
        assert np.array_equal(G.host(getattr(blk, n)), single[n]), "side stream: %s" % n
    ref = _oracle_block(x, w1, w3, w2, dy, rowwise, e5m2)
    for name, qz in (("qx", blk.qx), ("q1", blk.qw1), ("q3", blk.qw3), ("q2", blk.qw2)):
        G.assert_quantize_equal(_host_q(qz), ref[name], name)
    qx, q1, q3 = ref["qx"], ref["q1"], ref["q3"]
    G.gemm_parity(G.host(blk.a), ref["a"], qx[0], q1[0], qx[2], q1[2], label="block a")
    G.gemm_parity(G.host(blk.b), ref["b"], qx[0], q3[0], qx[2], q3[2], label="block b")
    for name in ("h", "out", "dh", "grad_w2", "da", "db", "grad_x", "grad_w1", "grad_w3"):
        got = G.host(getattr(blk, name))
        rf = oracle.rel_frobenius(got, ref[name])
        G.say("block", name, "relfro", rf)
        assert np.all(np.isfinite(_value(got))), name
        assert rf <= 1e-2, "%s: relative Frobenius %.3g" % (name, rf)
