"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from float8_mixed_precision_amd import ops
from float8_mixed_precision_amd import workloads as W
from tests import mfma_model as MM

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


def gemm_parity(G, O, a, b, sa, sb, ii=None, jj=None, label="", frob_tol=1e-3, e5m2_a=False):
    """Compare GPU bf16 outputs G with the oracle's O (same fp8 inputs).

    Required: relative Frobenius <= frob_tol and, for every element,
    |G - O| <= 2 ulp_bf16(O) + inv_a inv_b D(i, j) (1 + 2^-20), with D the
    largest distance between the oracle's sequential fp32 accumulator and
    the instruction's (tests/mfma_model.py, where the bound is derived from
    the reading of the instruction's accumulation).  Also reported: the
    share of elements within 2 bf16 ulps and the largest ulp distance."""
    G = np.asarray(G, np.uint16).ravel()
    O = np.asarray(O, np.uint16).ravel()
    m, k = a.shape
    n = b.shape[0]
    if ii is None:
        ii, jj = np.divmod(np.arange(m * n), n)
    ii = np.asarray(ii)
    jj = np.asarray(jj)
    sa = np.atleast_1d(sa).astype(np.float32)
    sb = np.atleast_1d(sb).astype(np.float32)
    inva = (np.float32(1) / sa).astype(np.float64)
    invb = (np.float32(1) / sb).astype(np.float64)
    inva = inva[ii] if inva.size > 1 else np.full(len(ii), inva[0])
    invb = invb[jj] if invb.size > 1 else np.full(len(jj), invb[0])
    dmax = MM.sum_difference_bound(a, b, ii, jj, e5m2_a)
    g = oracle.bf16_to_f32(G).astype(np.float64)
    o = oracle.bf16_to_f32(O).astype(np.float64)
    nxt = oracle.bf16_to_f32((O & 0x7FFF) + 1).astype(np.float64)
    ulp = np.abs(nxt - np.abs(o))
    allowed = 2 * ulp + inva * invb * dmax * (1 + 2.0 ** -20)
    err = np.abs(g - o)
    dist = oracle.bf16_ulp_distance(G, O)
    rf = oracle.rel_frobenius(G, O)
    stats = dict(n=len(G), relfro=rf, max_ulp=int(dist.max()) if len(dist) else 0,
                 frac_le2=float(np.mean(dist <= 2)) if len(dist) else 1.0,
                 max_bound_use=float(np.max(err / np.where(allowed > 0, allowed, np.inf)))
                 if len(err) else 0.0)
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
