"""GPU parity of the quantize path (amax -> scale -> saturating E4M3 cast and
transpose) against the oracle: bytes and scales bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from float8_mixed_precision_amd import ops
from float8_mixed_precision_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def test_encode_band_exhaustive():
    """Device conversion on every positive fp32 pattern of exponents 115..136
    (where E4M3 rounding happens), and their negatives."""
    for e in range(115, 137, 2):
        G.say("encode exponents", e, e + 1)
        bits = np.arange(e << 23, (e + 2) << 23, dtype=np.uint32)
        y = bits.view(np.float32)
        yd = torch.from_numpy(y).to(G.DEV)
        got = G.host(ops.fp8_linear_encode_e4m3(yd))
        want = oracle.e4m3_encode(y)
        assert np.array_equal(got, want), "exponent %d" % e
        got_neg = G.host(ops.fp8_linear_encode_e4m3(-yd))
        assert np.array_equal(got_neg, want ^ 0x80), "negative, exponent %d" % e


def test_encode_random_and_special():
    rng = np.random.default_rng(21)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000,
                        1, 0x80000001, 0x7F7FFFFF, 0xFF7FFFFF, 0x43E00000, 0x43E80000,
                        0x3A800000, 0x3AC00000], np.uint32)
    y = np.concatenate([bits, special]).view(np.float32)
    for n in (y.size, 3, 1):          # also tails that are not a multiple of 4
        G.say("encode random", n)
        got = G.host(ops.fp8_linear_encode_e4m3(torch.from_numpy(y[:n].copy()).to(G.DEV)))
        want = oracle.e4m3_encode(y[:n])
        nan = np.isnan(y[:n])
        assert np.all((got[nan] & 0x7F) == 0x7F)
        assert np.array_equal(got[~nan], want[~nan])


def all_finite_bf16(rows=256):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = (h & 0x7F80) != 0x7F80
    h = np.where(fin, h, 0).astype(np.uint16)
    return h.reshape(rows, -1)


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_quantize_every_bf16_value(rowwise):
    """Every finite bf16 pattern, with the largest magnitude forced to several
    levels so that the scaled values sweep the whole E4M3 range, including
    subnormal results and bf16 subnormal inputs."""
    base = all_finite_bf16()
    f = oracle.bf16_to_f32(base)
    for lim in (3.0e38, 1e5, 448.0, 1.0, 1e-3, 1e-30, 1e-38):
        x = np.where(np.abs(f) <= lim, base, 0).astype(np.uint16)
        G.say("quantize all-bf16 lim", lim, "rowwise", rowwise)
        got = G.gpu_quantize(x, rowwise)
        ref = oracle.quantize(x, rowwise)
        G.assert_quantize_equal(got, ref, "all-bf16 lim %g" % lim)
        # transposed layout too (rows and columns swap roles)
        got = G.gpu_quantize(np.ascontiguousarray(x.T), rowwise)
        ref = oracle.quantize(np.ascontiguousarray(x.T), rowwise)
        G.assert_quantize_equal(got, ref, "all-bf16^T lim %g" % lim)


SHAPES = [(16, 16), (256, 256), (272, 400), (48, 4112), (1040, 80), (528, 784), (144, 2064)]


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%d" % s)
def test_quantize_shapes(shape, rowwise):
    """Ragged shapes (not multiples of the 64x256 amax or 128x128 cast tiles)
    and several distributions."""
    rng = np.random.default_rng(hash(shape) % 1000)
    cases = {
        "normal": W.random_bf16(3, shape, 1.0, 0),
        "weights": W.random_bf16(3, shape, 0.02, 1),
        "student_t": W.to_bf16_bits(rng.standard_t(3, size=shape).astype(np.float32)),
    }
    for name, x in cases.items():
        G.say("quantize", shape, name, "rowwise", rowwise)
        G.assert_quantize_equal(G.gpu_quantize(x, rowwise), oracle.quantize(x, rowwise),
                                "%s %s" % (shape, name))



@pytest.mark.parametrize("offset", [0, 1, 2, 3], ids=lambda o: "scale+%dB" % (4 * o))
def test_quantize_rowwise_scale_alignment(offset):
    """Rowwise scale vectors at every 4-byte alignment (the interface requires
    4; 16-byte aligned ones are read as float4, the others one by one): the
    same bytes and scales as the oracle."""
    rows, cols = 272, 400
    x = W.random_bf16(5, (rows, cols), 1.0, 0)
    sbuf = torch.zeros(rows + 8, dtype=torch.float32, device=G.DEV)
    stbuf = torch.zeros(cols + 8, dtype=torch.float32, device=G.DEV)
    qz = ops.Quantized(torch.empty((rows, cols), dtype=torch.uint8, device=G.DEV),
                       torch.empty((cols, rows), dtype=torch.uint8, device=G.DEV),
                       sbuf[offset:offset + rows], stbuf[offset:offset + cols],
                       torch.empty(rows + cols, dtype=torch.float32, device=G.DEV))
    G.say("quantize rowwise, scale vectors offset by", 4 * offset, "bytes")
    ops.fp8_linear_quantize(G.dev_bf16(x), True, out=qz)
    torch.cuda.synchronize()
    got = (G.host(qz.q), G.host(qz.qt), G.host(qz.scale), G.host(qz.scale_t), G.host(qz.amax))
    G.assert_quantize_equal(got, oracle.quantize(x, True), "scale offset %d" % offset)


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_quantize_special_tensors(rowwise):
    shape = (272, 400)
    rng = np.random.default_rng(5)
    x = W.random_bf16(4, shape, 1.0, 2)
    cases = {}
    cases["zeros"] = np.zeros(shape, np.uint16)
    one = np.zeros(shape, np.uint16)
    one[100, 37] = 0x3F80
    cases["single"] = one
    cases["constant"] = np.full(shape, 0xC0A0, np.uint16)
    big = x.copy()
    big[7, 300] = 0x7F00                                   # ~1.7e38 outlier
    cases["outlier"] = big
    sub = x.copy()
    sub[:32] = W.to_bf16_bits(rng.standard_normal((32, shape[1])).astype(np.float32) * 1e-39)
    cases["subnormal_rows"] = sub
    zr = x.copy()
    zr[16:32] = 0
    zr[:, 64:80] = 0
    zr[200] = 0x8000                                       # a row of -0
    cases["zero_rows_cols"] = zr
    neg = x.copy()
    neg[np.abs(oracle.bf16_to_f32(neg)) < 0.5] = 0x8000
    cases["neg_zeros"] = neg
    for name, c in cases.items():
        G.say("quantize special", name, "rowwise", rowwise)
        G.assert_quantize_equal(G.gpu_quantize(c, rowwise), oracle.quantize(c, rowwise), name)


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_quantize_non_finite_surfaces_in_amax(rowwise):
    """NaN / inf inputs are no error: they must show up in amax (and not
    crash); the bytes are unspecified."""
    shape = (128, 256)
    x = W.random_bf16(6, shape, 1.0, 3)
    xn = x.copy()
    xn[5, 9] = 0x7FC0                                      # NaN
    xi = x.copy()
    xi[77, 200] = 0xFF80                                   # -inf
    G.say("quantize non-finite rowwise", rowwise)
    _, _, _, _, am = G.gpu_quantize(xn, rowwise)
    assert np.isnan(am[0] if not rowwise else am[5]) and (not rowwise or np.isnan(am[shape[0] + 9]))
    _, _, _, _, am = G.gpu_quantize(xi, rowwise)
    if rowwise:
        assert np.isposinf(am[77]) and np.isposinf(am[shape[0] + 200])
        assert np.all(np.isfinite(np.delete(am, [77, shape[0] + 200])))
    else:
        assert np.isposinf(am[0])


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
@pytest.mark.parametrize("shape", [(0, 0), (0, 32), (48, 0)], ids=lambda s: "%dx%d" % s)
def test_quantize_empty(shape, rowwise):
    """An empty matrix is valid: scales of the empty set (amax 0 ->
    448 / 1e-12), nothing else written."""
    G.say("quantize empty", shape, rowwise)
    x = torch.empty(shape, dtype=torch.bfloat16, device=G.DEV)
    qz = ops.fp8_linear_quantize(x, rowwise)
    torch.cuda.synchronize()
    s_empty = oracle.scale_from_amax(0.0)
    if rowwise:
        assert np.all(G.host(qz.scale) == s_empty) and np.all(G.host(qz.scale_t) == s_empty)
        assert np.all(G.host(qz.amax) == 0)
    else:
        assert G.host(qz.scale)[0] == s_empty and G.host(qz.amax)[0] == 0


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_quantize_workspace_reuse(rowwise):
    """One workspace serves calls of different sizes in a row (stale partial
    maxima of a bigger earlier call must not leak into a smaller one), and
    each result is bit-exact."""
    shapes = [(1040, 4112), (272, 400), (2064, 2064), (16, 16), (1040, 4112)]
    need = max(ops.fp8_linear_workspace_bytes(r, c, rowwise) for r, c in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=G.DEV)   # large stale maxima
    for k, shape in enumerate(shapes):
        x = W.random_bf16(30 + k, shape, 1.0, 5)
        G.say("quantize workspace reuse", shape, "rowwise", rowwise)
        G.assert_quantize_equal(G.gpu_quantize(x, rowwise, workspace=ws),
                                oracle.quantize(x, rowwise), "%s call %d" % (shape, k))


def test_quantize_scaled_max_maps_to_448():
    """Invariant on the device: the element(s) holding the amax encode to
    +-448 (0x7E / 0xFE)."""
    x = W.random_bf16(7, (528, 784), 1.0, 4)
    f = oracle.bf16_to_f32(x)
    q, qt, s, st, am = G.gpu_quantize(x, False)
    hit = np.abs(f) == np.abs(f).max()
    assert np.all((q[hit] & 0x7F) == 0x7E) and np.all((qt.T[hit] & 0x7F) == 0x7E)
    q, qt, s, st, am = G.gpu_quantize(x, True)
    assert np.all((q[np.abs(f) == np.abs(f).max(axis=1, keepdims=True)] & 0x7F) == 0x7E)
    assert np.all((qt.T[np.abs(f) == np.abs(f).max(axis=0, keepdims=True)] & 0x7F) == 0x7E)


@pytest.mark.parametrize("rowwise", [False, True], ids=["tensorwise", "rowwise"])
def test_quantize_beyond_2_31_elements(rowwise):
    """A quantize of bf16 [65536, 32768] (2^31 elements, 4 GiB): element
    offsets pass 2^31, so the 64-bit indexing of the amax passes, the
    rowwise finalize and the cast is exercised.  Sampled rows of q and of
    qT (first, last and random) and their scales match the oracle bit for
    bit.  Tensorwise: the oracle's scale of the host amax and its cast of
    those elements with that scale.  Rowwise: a row's q and row scale are
    the oracle's rowwise quantize of that row alone, and a column's qT and
    column scale that of the column alone."""
    R, C, B = 65536, 32768, 4096
    rng = np.random.default_rng(95)
    # bf16 patterns with random sign and mantissa, exponents 2^-7 .. 2^0: a
    # random [4096, C] block repeated down the rows (row r holds block row
    # r % 4096), so the host side stays cheap at this size
    blk = rng.integers(0, 1 << 16, size=(B, C), dtype=np.uint16)
    blk = (blk & 0x807F) | ((120 + ((blk >> 7) & 7)) << 7).astype(np.uint16)
    x = np.tile(blk, (R // B, 1))
    G.say("quantize beyond 2^31 elements", (R, C), "rowwise", rowwise)
    xd = G.dev_bf16(x)
    qz = ops.fp8_linear_quantize(xd, rowwise)
    torch.cuda.synchronize()
    del xd
    rows = np.unique(np.concatenate([[0, R - 2, R - 1], rng.integers(0, R, 13)]))
    cols = np.unique(np.concatenate([[0, C - 2, C - 1], rng.integers(0, C, 13)]))
    q_rows = G.host(qz.q[torch.as_tensor(rows, device=G.DEV)])
    qt_rows = G.host(qz.qt[torch.as_tensor(cols, device=G.DEV)])
    f32 = lambda v: np.asarray(v, np.float32).view(np.uint32)
    if not rowwise:
        amax_bits = int((blk & 0x7FFF).max())
        amax = np.float32(np.asarray(oracle.bf16_to_f32(np.array([amax_bits], np.uint16))).ravel()[0])
        s = np.float32(oracle.scale_from_amax(amax))
        assert f32(G.host(qz.scale))[0] == f32(s), (G.host(qz.scale)[0], s)
        assert np.array_equal(q_rows, oracle.quantize_scaled(blk[rows % B], s)[0]), "q rows"
        col_bits = np.ascontiguousarray(np.tile(blk[:, cols].T, (1, R // B)))
        assert np.array_equal(qt_rows, oracle.quantize_scaled(col_bits, s)[0]), "qT rows"
        return
    scale, scale_t = G.host(qz.scale), G.host(qz.scale_t)
    for i, r in enumerate(rows):
        q1, _, s1, _, _ = oracle.quantize(blk[[r % B]], True)
        assert np.array_equal(q_rows[i], q1[0]), "q row %d" % r
        assert f32(scale[r]) == f32(s1[0]), ("row scale", r)
    for i, c in enumerate(cols):
        col = np.ascontiguousarray(np.tile(blk[:, c], R // B).reshape(R, 1))
        _, qt1, _, st1, _ = oracle.quantize(col, True)
        assert np.array_equal(qt_rows[i], qt1[0]), "qT row %d" % c
        assert f32(scale_t[c]) == f32(st1[0]), ("column scale", c)
