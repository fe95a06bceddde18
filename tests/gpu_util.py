"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from float8_mixed_precision_amd import ops
from float8_mixed_precision_amd import workloads as W

DEV = "cuda:0"
U = 2.0 ** -24


def say(*a):
    """Name the case before a GPU step (flushed, so a lost box still shows it)."""
    print("[gpu]", *a, file=sys.stderr, flush=True)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return W.bits_to_torch(bits, DEV)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.atleast_1d(a), dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def gpu_quantize(bits: np.ndarray, rowwise: bool, workspace=None):
    x = dev_bf16(bits)
    qz = ops.fp8_linear_quantize(x, rowwise, workspace=workspace)
    torch.cuda.synchronize()
    return host(qz.q), host(qz.qt), host(qz.scale), host(qz.scale_t), host(qz.amax)


def assert_quantize_equal(got, ref, label=""):
    names = ("q", "qt", "scale", "scale_t", "amax")
    for n, g, r in zip(names, got, ref):
        g = np.asarray(g)
        r = np.asarray(r)
        assert g.shape == r.shape, (label, n, g.shape, r.shape)
        if g.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            i = tuple(bad[0])
            raise AssertionError("%s: %s differs at %d positions, first %s: gpu %#x oracle %#x"
                                 % (label, n, len(bad), i, int(g[i]), int(r[i])))


def _abs_dot(a, b, tv, ii, jj, chunk=256, tvb=None):
    """sum_t |A[i,t]| |B[j,t]| in float64 for the sampled pairs (codes are
    decoded per chunk of samples, so full-size operands never expand); tv
    decodes A's codes and tvb (default tv) B's."""
    av = np.abs(np.nan_to_num(tv, nan=0.0, posinf=0.0, neginf=0.0))
    bv = av if tvb is None else np.abs(np.nan_to_num(tvb, nan=0.0, posinf=0.0, neginf=0.0))
    out = np.empty(len(ii), np.float64)
    for s in range(0, len(ii), chunk):
        x = av[a[ii[s:s + chunk]]]
        y = bv[b[jj[s:s + chunk]]]
        out[s:s + chunk] = np.einsum("ij,ij->i", x, y)
    return out


def gemm_parity(G, O, a, b, sa, sb, ii=None, jj=None, label="", frob_tol=1e-3, e5m2_a=False):
    """Compare GPU bf16 outputs G with the oracle's O (same fp8 inputs).

    Required: relative Frobenius <= frob_tol and, for every element,
    |G - O| <= 2 ulp_bf16(O) + |inv_a inv_b| 2 gamma_k (|A||B|)_ij, the room
    two valid fp32 summation orders can differ by.  Also reported: the share
    of elements within 2 bf16 ulps and the largest ulp distance."""
    G = np.asarray(G, np.uint16).ravel()
    O = np.asarray(O, np.uint16).ravel()
    m, k = a.shape
    n = b.shape[0]
    if ii is None:
        ii, jj = np.divmod(np.arange(m * n), n)
    sa = np.atleast_1d(sa).astype(np.float32)
    sb = np.atleast_1d(sb).astype(np.float32)
    inva = (np.float32(1) / sa).astype(np.float64)
    invb = (np.float32(1) / sb).astype(np.float64)
    inva = inva[ii] if inva.size > 1 else np.full(len(ii), inva[0])
    invb = invb[jj] if invb.size > 1 else np.full(len(jj), invb[0])
    tv = oracle.e4m3_values()
    ta = oracle.e5m2_values() if e5m2_a else tv
    absdot = _abs_dot(a, b, ta, np.asarray(ii), np.asarray(jj), tvb=tv)
    g = oracle.bf16_to_f32(G).astype(np.float64)
    o = oracle.bf16_to_f32(O).astype(np.float64)
    nxt = oracle.bf16_to_f32((O & 0x7FFF) + 1).astype(np.float64)
    ulp = np.abs(nxt - np.abs(o))
    gam = k * U / (1 - k * U)
    allowed = 2 * ulp + inva * invb * 2 * gam * absdot
    err = np.abs(g - o)
    dist = oracle.bf16_ulp_distance(G, O)
    rf = oracle.rel_frobenius(G, O)
    stats = dict(n=len(G), relfro=rf, max_ulp=int(dist.max()) if len(dist) else 0,
                 frac_le2=float(np.mean(dist <= 2)) if len(dist) else 1.0)
    say("parity", label, stats)
    assert np.all(np.isfinite(g)), "%s: non-finite GPU output" % label
    assert rf <= frob_tol, "%s: relative Frobenius %.3g > %.3g" % (label, rf, frob_tol)
    bad = err > allowed
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError("%s: %d elements outside the bound; first (%d,%d): gpu %r oracle %r"
                             % (label, int(bad.sum()), ii[i], jj[i], g[i], o[i]))
    return stats


def sample_indices(m, n, count, seed, tile=256):
    """Random output positions plus the corners of every tile row/column
    boundary and the ragged last row/column."""
    rng = np.random.default_rng(seed)
    ii = list(rng.integers(0, m, count))
    jj = list(rng.integers(0, n, count))
    edges_m = sorted({0, m - 1} | {min(m - 1, t) for t in range(tile - 1, m, tile)}
                     | {min(m - 1, t) for t in range(tile, m, tile)})
    edges_n = sorted({0, n - 1} | {min(n - 1, t) for t in range(tile - 1, n, tile)}
                     | {min(n - 1, t) for t in range(tile, n, tile)})
    for i in edges_m[:64]:
        for j in edges_n[:64]:
            ii.append(i)
            jj.append(j)
    return np.array(ii, np.int64), np.array(jj, np.int64)
