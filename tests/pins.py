"""Pins for the CPU oracle: checks against things other than the oracle.

Each check takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  What each check compares against:

* torch's CPU float8_e4m3fn / bfloat16 conversions (library routines that
  share nothing with oracle.c);
* facts of the E4M3 format of the FP8 formats paper named on the
  "torchtitan" tutorial page (Part XI, item 9): 448 largest finite value,
  2^-6 smallest normal, 2^-9 smallest subnormal, NaN only at S.1111.111;
* brute-force nearest-value search over all finite codes in float64;
* exact float64 sums (every fp8 x fp8 product is a multiple of 2^-18 below
  2^18, so sums of fewer than 2^16 of them are exact in float64) and the
  standard bound |fl(sum) - sum| <= gamma_k * sum |terms| for recursive fp32
  summation;
* invariants (a scaled maximum maps to 448, zero maps to zero, sign symmetry,
  monotonicity, permutation equivariance).
"""
from __future__ import annotations

import numpy as np
import torch

U = 2.0 ** -24          # unit roundoff of fp32


# ------------------------------------------------------------- helpers --

def torch_e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 codes, decoded by torch."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()


def torch_encode_sat(y: np.ndarray) -> np.ndarray:
    """Saturating e4m3 encode via torch: clamp to +-448, then torch's RNE cast
    (torch's own cast is non-saturating, so the clamp comes first)."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_bf16_bits(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_from_bits(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def brute_force_encode(y: np.ndarray, tv: np.ndarray) -> np.ndarray:
    """Nearest finite code by exhaustive scan of the magnitudes of codes
    0x00..0x7E (values from torch), ties to the even code, saturating at
    448, sign bit from y, NaN -> NaN code.  Pure brute force, no bisection."""
    y = np.asarray(y, dtype=np.float32)
    mags = tv[:0x7F]                                  # codes 0..126
    m = np.abs(y.astype(np.float64))
    d = np.abs(m[:, None] - mags[None, :])            # [n, 127]
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(0x7F)
    # among equidistant codes prefer the even one
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    pick = np.where(m >= 448.0, 0x7E, pick)
    sign = np.signbit(y).astype(np.int64) << 7
    out = (pick | sign).astype(np.uint8)
    out = np.where(np.isnan(y), (0x7F | sign).astype(np.uint8), out)
    return out


def gamma(k: int) -> float:
    return k * U / (1.0 - k * U)


def random_codes(rng, shape, lo=0x00, hi=0x7E) -> np.ndarray:
    """Random finite codes with random signs."""
    mag = rng.integers(lo, hi + 1, size=shape)
    sign = rng.integers(0, 2, size=shape) << 7
    return (mag | sign).astype(np.uint8)


# ---------------------------------------------------------------- e4m3 --

def check_decode(o) -> None:
    ov = o.e4m3_values()
    tv = torch_e4m3_values()
    nan_o = np.isnan(ov)
    assert np.array_equal(nan_o, np.isnan(tv)), "NaN codes differ from torch"
    assert np.array_equal(np.flatnonzero(nan_o), [0x7F, 0xFF]), "NaN codes"
    assert np.array_equal(ov[~nan_o], tv[~nan_o]), "decoded values differ from torch"
    # facts of the E4M3 format
    assert ov[0x7E] == 448.0 and ov[0xFE] == -448.0
    assert ov[0x08] == 2.0 ** -6 and ov[0x01] == 2.0 ** -9
    assert ov[0x00] == 0.0 and np.signbit(ov[0x80])
    assert np.count_nonzero(np.isfinite(ov)) == 254
    assert np.all(np.diff(ov[:0x7F]) > 0), "positive codes not increasing"
    assert np.array_equal(ov[0x80:0xFF], -ov[0x00:0x7F])


def check_encode_band(o, exps=range(115, 137)) -> None:
    """Every positive fp32 pattern whose exponent lies where e4m3 rounding
    happens (2^-12 <= y < 2^10), one exponent (2^23 patterns) at a time,
    against torch's saturating cast."""
    for e in exps:
        bits = np.arange(e << 23, (e + 1) << 23, dtype=np.uint32)
        y = f32_from_bits(bits)
        a = o.e4m3_encode(y)
        b = torch_encode_sat(y)
        if not np.array_equal(a, b):
            i = int(np.flatnonzero(a != b)[0])
            raise AssertionError("encode(%r) = %#x, torch %#x"
                                 % (float(y[i]), a[i], b[i]))


def check_encode_random(o, n: int = 1 << 22, seed: int = 1) -> None:
    """Random fp32 patterns over the whole 2^32 range (both signs, all
    exponents, NaN and inf included) against torch; NaNs map to NaN codes."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000,
                         0x7FC00000, 0xFFC00000, 0x00000001, 0x80000001,
                         0x7F7FFFFF, 0xFF7FFFFF], dtype=np.uint32)
    y = f32_from_bits(np.concatenate([bits, specials]))
    a = o.e4m3_encode(y)
    nan = np.isnan(y)
    assert np.all((a[nan] & 0x7F) == 0x7F), "NaN must encode to a NaN code"
    b = torch_encode_sat(y[~nan])
    if not np.array_equal(a[~nan], b):
        i = int(np.flatnonzero(a[~nan] != b)[0])
        raise AssertionError("encode(%r) = %#x, torch %#x"
                             % (float(y[~nan][i]), a[~nan][i], b[i]))


def check_encode_brute_force(o, seed: int = 2) -> None:
    """Brute-force nearest value on random values, on every midpoint between
    adjacent codes and on its fp32 neighbours, on both signs."""
    tv = torch_e4m3_values()
    mags = tv[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2.0                 # exact in fp32
    mids32 = mids.astype(np.float32)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    rng = np.random.default_rng(seed)
    r = (rng.standard_normal(200_000) * rng.choice([1e-3, 1e-2, 1, 30, 300], 200_000)).astype(np.float32)
    extra = np.array([448, 464, 464.00003, 480, 1e6, np.inf, 2 ** -10, 2 ** -11,
                      1.5 * 2 ** -10, 0.0, 3e-39, 1e-45], dtype=np.float32)
    y = np.concatenate([mids32, up, dn, r, extra])
    y = np.concatenate([y, -y])
    a = o.e4m3_encode(y)
    b = brute_force_encode(y, tv)
    if not np.array_equal(a, b):
        i = int(np.flatnonzero(a != b)[0])
        raise AssertionError("encode(%r) = %#x, brute force %#x" % (float(y[i]), a[i], b[i]))


def check_encode_invariants(o, seed: int = 3) -> None:
    tv = torch_e4m3_values()
    finite = np.flatnonzero(np.isfinite(tv))
    # round trip on every finite code
    rt = o.e4m3_encode(tv[finite].astype(np.float32))
    assert np.array_equal(rt, finite.astype(np.uint8)), "enc(dec(c)) != c"
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal(100_000) * 100).astype(np.float32)
    # sign symmetry
    assert np.array_equal(o.e4m3_encode(-y), o.e4m3_encode(y) ^ 0x80)
    # monotone: sorted inputs give non-decreasing decoded values
    ys = np.sort(np.abs(y))
    dv = tv[o.e4m3_encode(ys)]
    assert np.all(np.diff(dv) >= 0), "encode not monotone"
    # zero maps to zero, saturation at 448 and beyond
    z = o.e4m3_encode(np.array([0.0, -0.0], np.float32))
    assert z[0] == 0x00 and z[1] == 0x80
    s = o.e4m3_encode(np.array([448, 449, 1e30, np.inf, -448, -1e30, -np.inf], np.float32))
    assert np.array_equal(s, [0x7E] * 4 + [0xFE] * 3)


# ---------------------------------------------------------------- bf16 --

def check_bf16(o, seed: int = 4) -> None:
    # widening: all 65536 patterns against torch
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    a = o.bf16_to_f32(h)
    b = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(b)
    assert np.array_equal(np.isnan(a), nan)
    assert np.array_equal(a[~nan].view(np.uint32), b[~nan].view(np.uint32))
    # narrowing: random patterns, exact ties, overflow boundary, specials
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    hi = rng.integers(0, 1 << 16, size=1 << 16, dtype=np.uint64).astype(np.uint32) << 16
    ties = hi | 0x8000
    near = np.concatenate([ties - 1, ties + 1])
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x7F800000,
                     0xFF7F8000, 0xFF7FFFFF, 0x00008000, 0x00018000, 0x80008000,
                     0x7FC00000, 0xFFC00001, 0x00000001, 0x80000000], np.uint32)
    v = f32_from_bits(np.concatenate([bits, ties, near, edge]))
    a = o.f32_to_bf16(v)
    b = torch_bf16_bits(v)
    nan = np.isnan(v)
    assert np.all((a[nan] & 0x7FFF) > 0x7F80), "NaN must stay NaN"
    if not np.array_equal(a[~nan], b[~nan]):
        i = int(np.flatnonzero(a[~nan] != b[~nan])[0])
        raise AssertionError("bf16(%r) = %#x, torch %#x" % (float(v[~nan][i]), a[~nan][i], b[~nan][i]))


# ------------------------------------------------------------ quantize --

def _independent_quantize(xb: np.ndarray, rowwise: bool):
    """The same definitions through library routines: numpy max of |x|,
    float64 division rounded once to fp32 (a correctly rounded fp32 quotient,
    since 53 >= 2*24 + 2), torch fp32 multiply and torch's saturating cast."""
    x = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).float()
    ax = x.abs().numpy()
    eps = np.float64(np.float32(1e-12))

    def sc(a):
        a = np.asarray(a, np.float64)
        return (448.0 / np.maximum(a, eps)).astype(np.float32)

    if not rowwise:
        a = np.float32(ax.max()) if ax.size else np.float32(0)
        s = sc(a)
        q = torch_encode_sat((x * torch.tensor(s)).numpy())
        return q, q.T.copy(), np.array([s]), np.array([s]), np.array([a])
    ar = ax.max(axis=1)
    ac = ax.max(axis=0)
    sr, scol = sc(ar), sc(ac)
    q = torch_encode_sat((x * torch.from_numpy(sr)[:, None]).numpy())
    qt = torch_encode_sat((x * torch.from_numpy(scol)[None, :]).numpy()).T.copy()
    return q, qt, sr, scol, np.concatenate([ar, ac]).astype(np.float32)


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def check_quantize_vs_library(o, shapes=((64, 48), (128, 272), (37, 5)), seed=5) -> None:
    from float8_mixed_precision_amd.workloads import random_bf16, to_bf16_bits
    rng = np.random.default_rng(seed)
    for si, shp in enumerate(shapes):
        cases = [random_bf16(seed, shp, 1.0, si),
                 random_bf16(seed, shp, 0.02, si + 10),
                 to_bf16_bits(rng.standard_t(3, size=shp).astype(np.float32)
                              * np.where(rng.random(shp[1]) < 0.05, 100, 1).astype(np.float32))]
        for xb in cases:
            for rowwise in (False, True):
                got = o.quantize(xb, rowwise)
                ref = _independent_quantize(xb, rowwise)
                names = ("q", "qt", "scale", "scale_t", "amax")
                for n, g, r in zip(names, got, ref):
                    g = np.asarray(g)
                    r = np.asarray(r)
                    if g.dtype == np.float32:
                        g, r = _bits(g), _bits(r)
                    assert g.shape == r.shape, (n, g.shape, r.shape)
                    if not np.array_equal(g, r):
                        raise AssertionError("%s differs (shape %s rowwise %s)" % (n, shp, rowwise))


def check_scale(o, seed: int = 6) -> None:
    """scale = 448 / max(a, 1e-12) correctly rounded, over random amax."""
    rng = np.random.default_rng(seed)
    a = np.concatenate([
        (10.0 ** rng.uniform(-14, 6, 20000)).astype(np.float32),
        np.array([0.0, 1e-12, 5e-13, 448.0, 1.0, 3.0, 7.0], np.float32)])
    got = np.array([o.scale_from_amax(v) for v in a], np.float32)
    ref = (448.0 / np.maximum(a.astype(np.float64), np.float64(np.float32(1e-12)))).astype(np.float32)
    assert np.array_equal(_bits(got), _bits(ref)), "scale not the correctly rounded quotient"


def check_quantize_invariants(o, seed: int = 7) -> None:
    from float8_mixed_precision_amd.workloads import random_bf16
    xb = random_bf16(seed, (96, 80), 1.0, 0)
    x = o.bf16_to_f32(xb)
    # tensorwise: the amax element(s) map to +-448, qt is q transposed
    q, qt, s, st, am = o.quantize(xb, False)
    assert am[0] == np.abs(x).max() and s[0] == st[0]
    hit = np.abs(x) == am[0]
    assert np.all((q[hit] & 0x7F) == 0x7E)
    assert np.array_equal(qt, q.T)
    # rowwise: each row's / column's max maps to +-448
    q, qt, s, st, am = o.quantize(xb, True)
    rmax = np.abs(x).max(axis=1)
    cmax = np.abs(x).max(axis=0)
    assert np.array_equal(am, np.concatenate([rmax, cmax]))
    assert np.all((q[np.abs(x) == rmax[:, None]] & 0x7F) == 0x7E)
    assert np.all((qt.T[np.abs(x) == cmax[None, :]] & 0x7F) == 0x7E)
    # zero tensor: zero codes, scale 448 / 1e-12
    z = np.zeros((16, 32), np.uint16)
    q, qt, s, st, am = o.quantize(z, False)
    assert not q.any() and not qt.any() and am[0] == 0
    assert s[0] == np.float32(448.0 / np.float64(np.float32(1e-12)))
    # constant tensor c: every code is +-448
    c = np.full((16, 32), 0xC0A0, np.uint16)          # bf16 -5.0
    q, qt, s, st, am = o.quantize(c, True)
    assert np.all(q == 0xFE) and np.all(qt == 0xFE)


# ---------------------------------------------------------------- GEMM --

def _exact_sum(a, b, tv):
    """float64 A.B^T of decoded codes: exact for k < 2^16."""
    return tv[a] @ tv[b].T


def check_gemm_vs_exact(o, shapes=((24, 40, 300), (16, 16, 4096), (8, 12, 14336)), seed=8) -> None:
    """fp32 sums within gamma_k * sum|terms| of the exact float64 sums."""
    tv = torch_e4m3_values()
    rng = np.random.default_rng(seed)
    for (m, n, k) in shapes:
        a = random_codes(rng, (m, k))
        b = random_codes(rng, (n, k))
        out, acc = o.gemm_tn(a, np.float32(1.0), b, np.float32(1.0), return_acc=True)
        ex = _exact_sum(a, b, tv)
        bound = gamma(k) * (np.abs(tv[a]) @ np.abs(tv[b]).T)
        err = np.abs(acc.astype(np.float64) - ex)
        assert np.all(err <= bound), "fp32 sum outside gamma_k bound (%s)" % ((m, n, k),)
        # unit scales: output is the bf16 rounding of the fp32 sum
        assert np.array_equal(out, torch_bf16_bits(acc))


def check_gemm_exact_cases(o, seed: int = 9) -> None:
    """Codes whose partial sums are all exact in fp32 (values in [1, 16),
    k = 64: every partial sum is a multiple of 2^-6 below 2^14): the fp32
    sum must equal the exact sum bit for bit, and with power-of-two scales the
    output is bf16(exact / (sa * sb)) exactly."""
    tv = torch_e4m3_values()
    rng = np.random.default_rng(seed)
    m, n, k = 12, 20, 64
    a = random_codes(rng, (m, k), 0x38, 0x57)        # [1, 16)
    b = random_codes(rng, (n, k), 0x38, 0x57)
    sa = (2.0 ** rng.integers(-4, 5, m)).astype(np.float32)
    sb = (2.0 ** rng.integers(-4, 5, n)).astype(np.float32)
    out, acc = o.gemm_tn(a, sa, b, sb, return_acc=True)
    ex = _exact_sum(a, b, tv)
    assert np.array_equal(acc.astype(np.float64), ex)
    want = torch_bf16_bits((ex / (sa[:, None].astype(np.float64) * sb[None, :])).astype(np.float32))
    assert np.array_equal(out, want)


def check_gemm_scales(o, seed: int = 10) -> None:
    """General scales: the output is within one bf16 ulp of the exact value
    exact_sum / (sa_i * sb_j) rounded to bf16 (two fp32 reciprocals and two
    fp32 products add at most a few fp32 ulps before the bf16 rounding), and
    permuting rows of A together with sa permutes the output rows (and the
    same for B, sb and columns)."""
    from oracle import bf16_ulp_distance
    tv = torch_e4m3_values()
    rng = np.random.default_rng(seed)
    m, n, k = 33, 47, 200
    a = random_codes(rng, (m, k))
    b = random_codes(rng, (n, k))
    sa = (10.0 ** rng.uniform(-2, 4, m)).astype(np.float32)
    sb = (10.0 ** rng.uniform(-2, 4, n)).astype(np.float32)
    out = o.gemm_tn(a, sa, b, sb)
    ex = _exact_sum(a, b, tv) / (sa[:, None].astype(np.float64) * sb[None, :])
    want = torch_bf16_bits(ex.astype(np.float32))
    cancel = np.abs(_exact_sum(a, b, tv)) < 1e-3 * (np.abs(tv[a]) @ np.abs(tv[b]).T)
    d = bf16_ulp_distance(out, want)
    assert np.all(d[~cancel] <= 1), "epilogue more than 1 bf16 ulp off"
    pa = rng.permutation(m)
    pb = rng.permutation(n)
    out2 = o.gemm_tn(a[pa], sa[pa], b[pb], sb[pb])
    assert np.array_equal(out2, out[pa][:, pb])
    # a tensorwise call equals a rowwise call with constant vectors
    o1 = o.gemm_tn(a, np.float32(3.5), b, np.float32(0.25))
    o2 = o.gemm_tn(a, np.full(m, 3.5, np.float32), b, np.full(n, 0.25, np.float32))
    assert np.array_equal(o1, o2)


def check_gemm_tiny_brute_force(o, seed: int = 11) -> None:
    """Pure-Python triple loop in float64 on tiny shapes."""
    tv = torch_e4m3_values()
    rng = np.random.default_rng(seed)
    for (m, n, k) in ((1, 1, 1), (3, 5, 7), (4, 2, 33)):
        a = random_codes(rng, (m, k))
        b = random_codes(rng, (n, k))
        _, acc = o.gemm_tn(a, np.float32(1), b, np.float32(1), return_acc=True)
        for i in range(m):
            for j in range(n):
                s = 0.0
                t_abs = 0.0
                for t in range(k):
                    p = float(tv[a[i, t]]) * float(tv[b[j, t]])
                    s += p
                    t_abs += abs(p)
                assert abs(float(acc[i, j]) - s) <= gamma(k) * t_abs


def check_gemm_sampled(o, seed: int = 12) -> None:
    rng = np.random.default_rng(seed)
    m, n, k = 40, 30, 96
    a = random_codes(rng, (m, k))
    b = random_codes(rng, (n, k))
    sa = (rng.random(m) + 0.5).astype(np.float32)
    sb = (rng.random(n) + 0.5).astype(np.float32)
    full = o.gemm_tn(a, sa, b, sb)
    ii = rng.integers(0, m, 500)
    jj = rng.integers(0, n, 500)
    assert np.array_equal(o.gemm_tn_sampled(a, sa, b, sb, ii, jj), full[ii, jj])


def check_amax(o, seed: int = 13) -> None:
    """max |x| of a bf16 tensor against numpy on torch's bf16 decode: NaN
    propagates, the empty tensor gives 0, and it is the tensorwise quantize's
    amax."""
    from float8_mixed_precision_amd.workloads import random_bf16
    rng = np.random.default_rng(seed)
    for shp in ((64, 48), (7, 16), (1, 16)):
        xb = random_bf16(seed, shp, float(rng.uniform(0.01, 100)), 0)
        f = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
        assert np.float32(o.amax(xb)) == np.float32(np.abs(f).max())
        assert _bits(np.atleast_1d(o.amax(xb))) == _bits(o.quantize(xb, False)[4])
        xn = xb.copy()
        xn[shp[0] // 2, 3] = 0x7FC0
        assert np.isnan(o.amax(xn))
        for pos in ((0, 0), (shp[0] - 1, shp[1] - 1)):     # the first and the last element
            xe = xb.copy()
            xe[pos] = 0xC7C8                                  # -102400, the unique maximum |x|
            assert o.amax(xe) == np.float32(102400.0), "amax misses element %s" % (pos,)
    assert o.amax(np.zeros((0, 16), np.uint16)) == 0.0


def check_quantize_scaled(o, seed: int = 14) -> None:
    """Cast with a given scale against torch's saturating encode of the fp32
    product (numpy float32 multiply), over scales that keep, shrink and
    saturate the values; qt is q transposed; with the tensor's own scale it
    is the tensorwise quantize."""
    from float8_mixed_precision_amd.workloads import random_bf16
    for si, shp in enumerate(((64, 48), (37, 16), (128, 80))):
        xb = random_bf16(seed, shp, 1.0, si)
        f = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
        for s in (1.0, 3.7e-3, 55.0, 1e5, float(o.scale_from_amax(o.amax(xb)))):
            q, qt = o.quantize_scaled(xb, s)
            want = torch_encode_sat(f * np.float32(s))
            assert np.array_equal(q, want), "quantize_scaled q, scale %g" % s
            assert np.array_equal(qt, q.T)
        q0, qt0 = o.quantize(xb, False)[:2]
        q1, qt1 = o.quantize_scaled(xb, o.scale_from_amax(o.amax(xb)))
        assert np.array_equal(q0, q1) and np.array_equal(qt0, qt1)


def check_gemm_f32(o, seed: int = 15) -> None:
    """The fp32-output GEMM is the bf16 GEMM before its last rounding: its
    bf16 rounding (by torch) equals gemm_tn bit for bit, and with sums that
    are exact and power-of-two scales it equals exact / (sa * sb) exactly."""
    tv = torch_e4m3_values()
    rng = np.random.default_rng(seed)
    m, n, k = 33, 47, 200
    a = random_codes(rng, (m, k))
    b = random_codes(rng, (n, k))
    sa = (10.0 ** rng.uniform(-2, 4, m)).astype(np.float32)
    sb = (10.0 ** rng.uniform(-2, 4, n)).astype(np.float32)
    f = o.gemm_tn_f32(a, sa, b, sb)
    assert np.array_equal(torch_bf16_bits(f), o.gemm_tn(a, sa, b, sb))
    ii = rng.integers(0, m, 300)
    jj = rng.integers(0, n, 300)
    assert np.array_equal(_bits(o.gemm_tn_f32_sampled(a, sa, b, sb, ii, jj)), _bits(f[ii, jj]))
    m, n, k = 12, 20, 64
    a = random_codes(rng, (m, k), 0x38, 0x57)
    b = random_codes(rng, (n, k), 0x38, 0x57)
    sa = (2.0 ** rng.integers(-4, 5, m)).astype(np.float32)
    sb = (2.0 ** rng.integers(-4, 5, n)).astype(np.float32)
    ex = _exact_sum(a, b, tv) / (sa[:, None].astype(np.float64) * sb[None, :])
    assert np.array_equal(o.gemm_tn_f32(a, sa, b, sb).astype(np.float64), ex)


# ---------------------------------------------------------------- e5m2 --

def torch_e5m2_values() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e5m2).to(torch.float32).double().numpy()


def torch_encode_sat_e5m2(y: np.ndarray) -> np.ndarray:
    """Saturating E5M2 encode via torch: clamp to +-57344, then torch's RNE
    cast (which on its own overflows to inf)."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.clamp(-57344.0, 57344.0).to(torch.float8_e5m2).view(torch.uint8).numpy()


def check_e5m2_decode(o) -> None:
    """All 256 codes against torch's float8_e5m2, plus the format's facts:
    largest finite 57344, smallest normal 2^-14, smallest subnormal 2^-16,
    +-inf at S.11111.00, NaN at S.11111.{01,10,11}."""
    got = o.e5m2_values()
    ref = torch_e5m2_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7B] == 57344.0 and got[0x04] == 2.0 ** -14 and got[0x01] == 2.0 ** -16
    assert np.isposinf(got[0x7C]) and np.isneginf(got[0xFC])
    assert np.flatnonzero(nan).tolist() == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]


def check_e5m2_encode(o, n: int = 1 << 21, seed: int = 16) -> None:
    """Random fp32 patterns, values around every code and the rounding
    midpoints against torch's saturating cast; nearest-value brute force
    (ties to the even code) on a sample; sign symmetry."""
    rng = np.random.default_rng(seed)
    ev = torch_e5m2_values()
    fin = ev[:0x7C]
    mids = (fin[:-1] + fin[1:]) / 2
    y = np.concatenate([
        f32_from_bits(rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)),
        fin.astype(np.float32), mids.astype(np.float32),
        (mids * (1 + 2.0 ** -20)).astype(np.float32), (mids * (1 - 2.0 ** -20)).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 57344.0, 61440.0, 1e30, 2.0 ** -17, 2.0 ** -18,
                  3 * 2.0 ** -18], np.float32)])
    y = np.concatenate([y, -y])
    got = o.e5m2_encode(y)
    nan = np.isnan(y)
    assert np.all((got[nan] & 0x7F) > 0x7C), "NaN must give a NaN code"
    assert np.array_equal(got[~nan], torch_encode_sat_e5m2(y[~nan]))
    # brute force on a sample of finite values
    ys = y[~nan][rng.integers(0, int((~nan).sum()), 4000)]
    m = np.abs(ys.astype(np.float64))
    d = np.abs(m[:, None] - fin[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(fin.size)
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    pick = np.where(m >= 57344.0, 0x7B, pick)
    want = (pick | (np.signbit(ys).astype(np.int64) << 7)).astype(np.uint8)
    assert np.array_equal(o.e5m2_encode(ys), want)


def _independent_quantize_fmt(xb, rowwise, fmax, enc):
    """_independent_quantize for another format (largest finite fmax)."""
    x = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).float()
    ax = x.abs().numpy()
    eps = np.float64(np.float32(1e-12))

    def sc(a):
        return (fmax / np.maximum(np.asarray(a, np.float64), eps)).astype(np.float32)

    if not rowwise:
        a = np.float32(ax.max()) if ax.size else np.float32(0)
        s = sc(a)
        q = enc((x * torch.tensor(s)).numpy())
        return q, q.T.copy(), np.array([s]), np.array([s]), np.array([a])
    ar, ac = ax.max(axis=1), ax.max(axis=0)
    sr, scol = sc(ar), sc(ac)
    q = enc((x * torch.from_numpy(sr)[:, None]).numpy())
    qt = enc((x * torch.from_numpy(scol)[None, :]).numpy()).T.copy()
    return q, qt, sr, scol, np.concatenate([ar, ac]).astype(np.float32)


def check_quantize_e5m2(o, seed: int = 17) -> None:
    from float8_mixed_precision_amd.workloads import random_bf16
    for si, shp in enumerate(((64, 48), (37, 16), (128, 80))):
        for xb in (random_bf16(seed, shp, 1e-2, si), random_bf16(seed, shp, 3.0, si + 10)):
            for rowwise in (False, True):
                got = o.quantize_e5m2(xb, rowwise)
                ref = _independent_quantize_fmt(xb, rowwise, 57344.0, torch_encode_sat_e5m2)
                for name, g, r in zip(("q", "qt", "scale", "scale_t", "amax"), got, ref):
                    g, r = np.asarray(g), np.asarray(r)
                    if g.dtype == np.float32:
                        g, r = _bits(g), _bits(r)
                    assert g.shape == r.shape and np.array_equal(g, r), \
                        "e5m2 %s differs (shape %s rowwise %s)" % (name, shp, rowwise)


def check_gemm_mixed(o, seed: int = 18) -> None:
    """E5M2 x E4M3: (0, 0) is the pinned E4M3 GEMM; exact sums with
    power-of-two scales give bf16(exact / (sa sb)) exactly; general values
    stay within one bf16 ulp of the float64 value outside cancellations;
    sampled equals full."""
    from oracle import bf16_ulp_distance
    t4 = torch_e4m3_values()
    t5 = torch_e5m2_values()
    rng = np.random.default_rng(seed)
    m, n, k = 24, 40, 96
    a = random_codes(rng, (m, k))
    b = random_codes(rng, (n, k))
    sa = (rng.random(m) + 0.5).astype(np.float32)
    sb = (rng.random(n) + 0.5).astype(np.float32)
    assert np.array_equal(o.gemm_tn_mixed(a, 0, sa, b, 0, sb), o.gemm_tn(a, sa, b, sb))
    # exact: E5M2 values in [1, 8), E4M3 in [1, 16), k = 64
    a5 = random_codes(rng, (12, 64), 0x3C, 0x47)
    b4 = random_codes(rng, (20, 64), 0x38, 0x57)
    sa2 = (2.0 ** rng.integers(-4, 5, 12)).astype(np.float32)
    sb2 = (2.0 ** rng.integers(-4, 5, 20)).astype(np.float32)
    ex = (t5[a5] @ t4[b4].T) / (sa2[:, None].astype(np.float64) * sb2[None, :])
    assert np.array_equal(o.gemm_tn_mixed(a5, 1, sa2, b4, 0, sb2),
                          torch_bf16_bits(ex.astype(np.float32)))
    # general E5M2 codes (finite: magnitudes 0x00..0x7B)
    a5 = random_codes(rng, (m, k), 0x00, 0x7B)
    out = o.gemm_tn_mixed(a5, 1, sa, b, 0, sb)
    exact = t5[a5] @ t4[b].T
    want = torch_bf16_bits((exact / (sa[:, None].astype(np.float64) * sb[None, :])).astype(np.float32))
    cancel = np.abs(exact) < 1e-3 * (np.abs(t5[a5]) @ np.abs(t4[b]).T)
    assert np.all(bf16_ulp_distance(out, want)[~cancel] <= 1)
    ii = rng.integers(0, m, 300)
    jj = rng.integers(0, n, 300)
    assert np.array_equal(o.gemm_tn_mixed_sampled(a5, 1, sa, b, 0, sb, ii, jj), out[ii, jj])


# --------------------------------------------------------------- SwiGLU --

def _all_finite_bf16() -> np.ndarray:
    """Every finite bf16 bit pattern."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return bits[(bits & 0x7F80) != 0x7F80]


def _bf16_value64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _torch_silu_and_grad64(a64: np.ndarray):
    """silu and its derivative in float64 by torch (F.silu and autograd)."""
    t = torch.from_numpy(np.ascontiguousarray(a64, np.float64)).requires_grad_(True)
    y = torch.nn.functional.silu(t)
    y.sum().backward()
    return y.detach().numpy(), t.grad.numpy()


def check_silu(o, seed: int = 19) -> None:
    """silu on every finite bf16 input: the fp32 rounding of scipy's
    a * expit(a) and of torch's float64 F.silu; silu(0) = 0; silu(a) = a
    for large a, -> -0 for very negative a; silu(a) - silu(-a) = a within
    the two fp32 roundings; silu' equals torch's float64 autograd rounded to
    fp32 and a central difference of scipy's silu to 1e-6."""
    from scipy.special import expit
    a = _bf16_value64(_all_finite_bf16())
    a = a[np.abs(a) < 1e30]                       # keep the scipy product finite
    got = np.array([o.silu(v) for v in a[::7]], np.float32)
    want_sp = (a[::7] * expit(a[::7])).astype(np.float32)
    ts, tg = _torch_silu_and_grad64(a[::7])
    assert np.array_equal(got.view(np.uint32), want_sp.view(np.uint32)), "silu vs scipy"
    assert np.array_equal(got.view(np.uint32), ts.astype(np.float32).view(np.uint32)), \
        "silu vs torch"
    assert o.silu(0.0) == 0.0 and o.silu(100.0) == np.float32(100.0)
    assert o.silu(-1000.0) == 0.0 and np.signbit(o.silu(-1000.0))
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(2000) * 6).astype(np.float32)
    odd = np.array([float(o.silu(v)) - float(o.silu(-v)) for v in x])
    tol = 2 * np.spacing(np.abs(x)).astype(np.float64) + 1e-30
    assert np.all(np.abs(odd - x) <= tol), "silu(a) - silu(-a) != a"
    gd = np.array([o.dsilu(v) for v in a[::7]], np.float32)
    assert np.array_equal(gd.view(np.uint32), tg.astype(np.float32).view(np.uint32)), \
        "silu' vs torch autograd"
    xs = x.astype(np.float64)
    h = 1e-5 * np.maximum(1.0, np.abs(xs))
    f = lambda v: v * expit(v)
    fd = (f(xs + h) - f(xs - h)) / (2 * h)
    gx = np.array([o.dsilu(v) for v in x], np.float64)
    assert np.all(np.abs(gx - fd) <= 1e-6 * np.maximum(1.0, np.abs(fd))), "silu' vs difference"
    assert o.dsilu(0.0) == 0.5 and o.dsilu(1000.0) == 1.0


def check_swiglu_fwd(o, seed: int = 20) -> None:
    """h against torch: float64 F.silu rounded to fp32, an fp32 product with
    b, torch's bf16 rounding.  b = 1 gives bf16(silu(a)); b = 0 gives +-0;
    large a gives torch's bf16 product a*b; the order of a and b matters."""
    rng = np.random.default_rng(seed)
    from float8_mixed_precision_amd import workloads as W
    a = W.to_bf16_bits((rng.standard_normal((64, 96)) * 3).astype(np.float32))
    b = W.to_bf16_bits(rng.standard_normal((64, 96)).astype(np.float32))
    a[0, :4] = [0x0000, 0x8000, 0x7FC0, 0xFF80]                 # 0, -0, NaN, -inf
    a[1, :3] = [0x7F80, 0x42C8, 0xC2C8]                         # inf, 100, -100
    h = o.swiglu_fwd(a, b)
    s64, _ = _torch_silu_and_grad64(_bf16_value64(a))
    want = torch_bf16_bits(s64.astype(np.float32) * _bf16_value64(b).astype(np.float32))
    nan = np.isnan(_bf16_value64(want))
    assert np.array_equal(np.isnan(_bf16_value64(h)), nan)
    assert np.array_equal(h[~nan], want[~nan]), "swiglu fwd vs torch"
    one = np.full(a.shape, 0x3F80, np.uint16)
    assert np.array_equal(o.swiglu_fwd(a, one)[~nan], torch_bf16_bits(s64.astype(np.float32))[~nan])
    big = W.to_bf16_bits((rng.random((8, 16)) * 100 + 20).astype(np.float32))
    prod = torch_bf16_bits(_bf16_value64(big).astype(np.float32) * _bf16_value64(b[:8, :16]).astype(np.float32))
    assert np.array_equal(o.swiglu_fwd(big, b[:8, :16]), prod)
    zero = np.zeros(a.shape, np.uint16)
    fin = np.isfinite(_bf16_value64(a))
    assert np.all((o.swiglu_fwd(a, zero)[fin] & 0x7FFF) == 0)
    assert not np.array_equal(o.swiglu_fwd(b, a), h)


def check_swiglu_bwd(o, seed: int = 21) -> None:
    """da, db against torch autograd of F.silu(a) * b in float64: within one
    bf16 ulp of the exact gradients, and bit-equal to the exact gradients'
    factors combined in the stated fp32 order."""
    from oracle import bf16_ulp_distance
    from float8_mixed_precision_amd import workloads as W
    rng = np.random.default_rng(seed)
    shape = (48, 80)
    a = W.to_bf16_bits((rng.standard_normal(shape) * 3).astype(np.float32))
    b = W.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    dh = W.to_bf16_bits((rng.standard_normal(shape) * 1e-2).astype(np.float32))
    da, db = o.swiglu_bwd(dh, a, b)
    ta = torch.from_numpy(_bf16_value64(a)).requires_grad_(True)
    tb = torch.from_numpy(_bf16_value64(b)).requires_grad_(True)
    (torch.nn.functional.silu(ta) * tb).backward(torch.from_numpy(_bf16_value64(dh)))
    assert np.all(bf16_ulp_distance(da, torch_bf16_bits(ta.grad.numpy().astype(np.float32))) <= 1)
    assert np.all(bf16_ulp_distance(db, torch_bf16_bits(tb.grad.numpy().astype(np.float32))) <= 1)
    s64, g64 = _torch_silu_and_grad64(_bf16_value64(a))
    dh32 = _bf16_value64(dh).astype(np.float32)
    b32 = _bf16_value64(b).astype(np.float32)
    assert np.array_equal(da, torch_bf16_bits((dh32 * b32) * g64.astype(np.float32)))
    assert np.array_equal(db, torch_bf16_bits(dh32 * s64.astype(np.float32)))


def check_add_bf16(o, seed: int = 22) -> None:
    """bf16 + bf16 equals torch's CPU bf16 addition, finite and special."""
    rng = np.random.default_rng(seed)
    x = rng.integers(0, 1 << 16, 50000).astype(np.uint16)
    y = rng.integers(0, 1 << 16, 50000).astype(np.uint16)
    x[:6] = [0x7F80, 0xFF80, 0x7F80, 0x0001, 0x8000, 0x7F7F]
    y[:6] = [0xFF80, 0x3F80, 0x7F80, 0x8001, 0x8000, 0x7F7F]
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    ty = torch.from_numpy(y.view(np.int16)).view(torch.bfloat16)
    want = (tx + ty).view(torch.int16).numpy().view(np.uint16)
    got = o.add_bf16(x, y)
    nan = np.isnan(_bf16_value64(want))
    assert np.array_equal(np.isnan(_bf16_value64(got)), nan)
    assert np.array_equal(got[~nan], want[~nan])


ALL_CHECKS = [check_decode, check_encode_random, check_encode_brute_force,
              check_encode_invariants, check_bf16, check_scale,
              check_quantize_vs_library, check_quantize_invariants,
              check_gemm_vs_exact, check_gemm_exact_cases, check_gemm_scales,
              check_gemm_tiny_brute_force, check_gemm_sampled, check_amax,
              check_quantize_scaled, check_gemm_f32, check_e5m2_decode,
              check_e5m2_encode, check_quantize_e5m2, check_gemm_mixed, check_silu,
              check_swiglu_fwd, check_swiglu_bwd, check_add_bf16]
