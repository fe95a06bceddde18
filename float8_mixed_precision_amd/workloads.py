"""Seeded synthetic inputs for the Float8 linear layer.

This module is shared by the tests, the smoke check and the benchmark, and
feeds both the HIP path and the CPU oracle.  It holds none of the method's
arithmetic: it only draws random numbers with numpy, rounds them to bf16 with
torch's CPU conversion (the inputs of the layer are bf16 tensors, as in the
bf16 mixed-precision policy of the "torchtitan" tutorial page, Part IV,
Stage 5) and returns the bit patterns.

Shapes are those of a Llama-3.1 linear on one data-parallel rank: the
tutorial page's llama3_8b setup (Part II, "Using it") runs sequence length
8192 at a local batch of 1, so every linear sees M = 8192 token rows.  A
linear (M, N, K) has X [M, K] (activations, tokens x in-features),
W [N, K] (weights, out x in) and dY [M, N] (the output gradient).

Random streams: ``numpy.random.default_rng([seed, linear, t])`` with t = 0
for X, 1 for W, 2 for dY and 3 for the choice of outlier columns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Dist:
    kind: str            # "normal" or "student_t"
    sigma: float = 1.0   # standard deviation (normal)
    df: float = 3.0      # degrees of freedom (student_t)
    outlier_frac: float = 0.0   # fraction of columns multiplied by outlier_mul
    outlier_mul: float = 1.0


@dataclass(frozen=True)
class Linear:
    name: str
    M: int
    N: int
    K: int
    x: Dist
    w: Dist
    dy: Dist
    x_from: str = ""     # name of an earlier linear whose X this one shares


@dataclass(frozen=True)
class Workload:
    name: str
    rowwise: bool
    linears: Tuple[Linear, ...]
    seed: int = 0
    description: str = ""

    @property
    def flops(self) -> int:
        """Algorithmic flops of one fwd+bwd pass: 3 GEMMs of 2*M*N*K each."""
        return sum(6 * l.M * l.N * l.K for l in self.linears)


ACT = Dist("normal", 1.0)
WGT = Dist("normal", 0.02)
GRAD = Dist("normal", 1e-2)

WORKLOADS: Dict[str, Workload] = {
    "tiny_tw": Workload(
        "tiny_tw", False,
        (Linear("tiny", 256, 512, 256, ACT, WGT, Dist("normal", 1.0)),),
        description="tiny tensorwise linear: X[256x256] N(0,1), W[512x256] "
                    "N(0,0.02), dY[256x512] N(0,1)"),
    "attn8b_tw": Workload(
        "attn8b_tw", False,
        (Linear("attn_proj", 8192, 4096, 4096, ACT, WGT, GRAD),),
        description="Llama-3.1-8B attention projection, tensorwise: "
                    "X[8192x4096], W[4096x4096], dY[8192x4096]"),
    "ffn8b_tw": Workload(
        "ffn8b_tw", False,
        (Linear("w1", 8192, 14336, 4096, ACT, WGT, GRAD),
         Linear("w3", 8192, 14336, 4096, ACT, WGT, GRAD, x_from="w1"),
         Linear("w2", 8192, 4096, 14336, ACT, WGT, GRAD)),
        description="Llama-3.1-8B SwiGLU FFN, tensorwise: w1 and w3 "
                    "X[8192x4096].W[14336x4096]^T (shared X), w2 "
                    "X[8192x14336].W[4096x14336]^T; fwd+bwd per linear"),
    "ffn70b_tw": Workload(
        "ffn70b_tw", False,
        (Linear("w1", 8192, 28672, 8192, ACT, WGT, GRAD),),
        description="Llama-3.1-70B-shaped FFN linear on one GPU, tensorwise: "
                    "X[8192x8192], W[28672x8192], dY[8192x28672]"),
    "outlier_rw": Workload(
        "outlier_rw", True,
        (Linear("w1", 8192, 14336, 4096,
                Dist("student_t", df=3.0, outlier_frac=0.001, outlier_mul=100.0),
                WGT, GRAD),),
        description="rowwise-scaled outlier case at the 8B FFN shape: X "
                    "Student-t(3) with 0.1% of columns x100, W N(0,0.02), "
                    "dY N(0,1e-2); per-row / per-column scales"),
}


def _draw(rng: np.random.Generator, shape, d: Dist, rng_cols) -> np.ndarray:
    if d.kind == "normal":
        v = rng.standard_normal(shape, dtype=np.float32)
        if d.sigma != 1.0:
            v *= np.float32(d.sigma)
    elif d.kind == "student_t":
        v = rng.standard_t(d.df, size=shape).astype(np.float32)
    else:
        raise ValueError(d.kind)
    if d.outlier_frac > 0:
        ncols = shape[1]
        n_out = max(1, int(round(d.outlier_frac * ncols)))
        cols = np.sort(rng_cols.choice(ncols, size=n_out, replace=False))
        v[:, cols] *= np.float32(d.outlier_mul)
    return v


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp32 draws -> bf16 bit patterns (uint16), via torch's CPU rounding."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def tensor(seed: int, linear: int, t: int, shape, d: Dist) -> np.ndarray:
    rng = np.random.default_rng([seed, linear, t])
    rng_cols = np.random.default_rng([seed, linear, 3])
    return to_bf16_bits(_draw(rng, tuple(shape), d, rng_cols))


def generate_linear(w: Workload, li: int) -> Dict[str, np.ndarray]:
    """bf16 bit patterns {x, w, dy} of linear ``li`` of a workload."""
    l = w.linears[li]
    if l.x_from:
        src = [k for k, o in enumerate(w.linears) if o.name == l.x_from][0]
        x = tensor(w.seed, src, 0, (l.M, l.K), w.linears[src].x)
    else:
        x = tensor(w.seed, li, 0, (l.M, l.K), l.x)
    return {"x": x,
            "w": tensor(w.seed, li, 1, (l.N, l.K), l.w),
            "dy": tensor(w.seed, li, 2, (l.M, l.N), l.dy)}


def generate(w: Workload) -> List[Dict[str, np.ndarray]]:
    """bf16 bit patterns for every linear of a workload: [{x, w, dy}, ...].
    A linear whose X comes from an earlier one shares that array."""
    out: List[Dict[str, np.ndarray]] = []
    for li, l in enumerate(w.linears):
        if l.x_from:
            src = [k for k, o in enumerate(w.linears) if o.name == l.x_from][0]
            d = {"x": out[src]["x"],
                 "w": tensor(w.seed, li, 1, (l.N, l.K), l.w),
                 "dy": tensor(w.seed, li, 2, (l.M, l.N), l.dy)}
        else:
            d = generate_linear(w, li)
        out.append(d)
    return out


def random_bf16(seed: int, shape, sigma: float = 1.0, stream: int = 0) -> np.ndarray:
    """Plain N(0, sigma) bf16 bit patterns for ad-hoc test shapes."""
    return tensor(seed, 1000 + stream, 0, shape, Dist("normal", sigma))


def bits_to_torch(bits: np.ndarray, device=None) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor (copy)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(device) if device is not None else t
