"""Seeded synthetic inputs for the ternary GEMV/GEMM workloads.

Shared by the tests, the smoke check and the benchmark.  This module only
draws random numbers and describes shapes; it holds none of the method's
arithmetic (no packing, no quantization, no products).

Shapes follow a BitNet b1.58 2B-shaped transformer (hidden 2560, kv 640,
FFN 6912, 30 layers) and an 8B-shaped one (hidden 4096, kv 1024, FFN 14336,
32 layers).  Weights are [N, K] (out x in), activations [M, K].
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")

# (K, N) per projection: K = input features, N = output features.
SHAPES_2B = {"q": (2560, 2560), "k": (2560, 640), "v": (2560, 640),
             "o": (2560, 2560), "gate": (2560, 6912), "up": (2560, 6912),
             "down": (6912, 2560)}
SHAPES_8B = {"q": (4096, 4096), "k": (4096, 1024), "v": (4096, 1024),
             "o": (4096, 4096), "gate": (4096, 14336), "up": (4096, 14336),
             "down": (14336, 4096)}


@dataclass(frozen=True)
class WeightDist:
    p_neg: float
    p_zero: float  # P(+1) = 1 - p_neg - p_zero


UNIFORM = WeightDist(1 / 3, 1 / 3)
DECODE_2B = WeightDist(0.3, 0.4)
SKEWED_8B = WeightDist(0.2, 0.5)


def trits(rng: np.random.Generator, shape, dist: WeightDist = UNIFORM):
    """Ternary values in {-1, 0, +1} (int8) with the given probabilities."""
    if dist is UNIFORM:
        return rng.integers(-1, 2, size=shape, dtype=np.int8)
    u = rng.random(shape)
    out = np.ones(shape, np.int8)
    out[u < dist.p_neg + dist.p_zero] = 0
    out[u < dist.p_neg] = -1
    return out


def x_normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def x_normal_outliers(rng, shape, frac=0.01, mult=20.0):
    """N(0, 1) with each element independently multiplied by `mult` with
    probability `frac`."""
    x = rng.standard_normal(shape, dtype=np.float32)
    hit = rng.random(shape) < frac
    x[hit] *= np.float32(mult)
    return x


def x_student_t(rng, shape, nu=3.0):
    return rng.standard_t(nu, size=shape).astype(np.float32)


def scale(rng, lo, hi):
    return np.float32(rng.uniform(lo, hi))


# ---------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Problem:
    """One projection of one layer: weights [n, k] and activations [m, k]."""
    layer: int
    proj: str
    k: int
    n: int
    m: int


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    shapes: dict
    layers: int
    m: int
    dist: WeightDist
    s_lo: float
    s_hi: float
    x_kind: str  # "normal", "outliers", "student_t"
    projs: tuple = PROJ_NAMES

    def problems(self):
        return [Problem(l, p, self.shapes[p][0], self.shapes[p][1], self.m)
                for l in range(self.layers) for p in self.projs]

    def weight_bytes(self):
        return sum(p.n * p.k // 4 for p in self.problems())

    def rng_w(self, layer, proj):
        return np.random.default_rng(
            [self.seed, layer, PROJ_NAMES.index(proj), 0])

    def rng_x(self, layer, proj):
        return np.random.default_rng(
            [self.seed, layer, PROJ_NAMES.index(proj), 1, self.m])

    def weights(self, layer, proj):
        """(trits [n, k] int8, s_w float32) for one projection."""
        k, n = self.shapes[proj]
        rng = self.rng_w(layer, proj)
        t = trits(rng, (n, k), self.dist)
        return t, scale(rng, self.s_lo, self.s_hi)

    def activations(self, layer, proj, m=None):
        k, _ = self.shapes[proj]
        rng = self.rng_x(layer, proj)
        shape = (self.m if m is None else m, k)
        if self.x_kind == "outliers":
            return x_normal_outliers(rng, shape)
        if self.x_kind == "student_t":
            return x_student_t(rng, shape)
        return x_normal(rng, shape)


def decode_2b(m: int = 1, layers: int = 30) -> Workload:
    """2B-shaped decode set: 30 layers x 7 projections; P(0)=0.4,
    P(+-1)=0.3; s_w ~ U(0.01, 0.05); x N(0,1) with 1% outliers x20 (M=1),
    plain N(0,1) for the batched decode sizes M in {8, 16, 32}.  All M share
    the same weights (seed 2); activations are drawn per M."""
    return Workload(f"decode_2b_m{m}", 2, SHAPES_2B, layers,
                    m, DECODE_2B, 0.01, 0.05,
                    "outliers" if m == 1 else "normal")


def prefill_2b(m: int = 512) -> Workload:
    """One 2B-shaped layer, 7 projections, M=512, uniform trits."""
    return Workload(f"prefill_2b_m{m}", 4, SHAPES_2B, 1, m, UNIFORM, 0.01,
                    0.05, "normal")


def decode_8b(m: int = 1, layers: int = 32) -> Workload:
    """8B-shaped set: 32 layers x 7 projections; P(0)=0.5, P(+1)=0.3,
    P(-1)=0.2; s_w ~ U(0.005, 0.03); x Student-t (nu=3); M in {1, 64}."""
    return Workload(f"decode_8b_m{m}", 5, SHAPES_8B, layers, m, SKEWED_8B,
                    0.005, 0.03, "student_t")


# ----------------------------------------------------- layer-chained decode
# One token through the layers with every dependency kept: within a layer
# each phase quantizes an earlier output of the same layer (the layer input
# for the first phase) and runs the products that read it; the last output
# is the next layer's input.  Attention, the residual adds and the gated
# activation lie outside the ternary product, so the query output stands in
# for the attention output and the up output for the gated product.
CHAIN_PHASES = (("x", ("q", "k", "v")),
                ("q", ("o",)),
                ("o", ("gate", "up")),
                ("up", ("down",)))
CHAIN_OUT = "down"


def chain_input(work: Workload, m: int = 1):
    """The first layer's input for the layer-chained decode of a workload's
    weights: [m, hidden] drawn like that workload's activations."""
    rng = np.random.default_rng([work.seed, 1 << 20, 0, 1, m])
    shape = (m, work.shapes["q"][0])
    if work.x_kind == "outliers":
        return x_normal_outliers(rng, shape)
    if work.x_kind == "student_t":
        return x_student_t(rng, shape)
    return x_normal(rng, shape)


NORM_EPS = 1e-5  # RMSNorm eps of the chained decode with normalization


def norm_gain(work: Workload, layer: int, phase: int):
    """Per-feature RMSNorm gain of one phase input of the layer-chained
    decode (no trained gains exist here): U(0.5, 1.5), fp32, [k]."""
    src = CHAIN_PHASES[phase][0]
    k = work.shapes["q"][0] if src == "x" else work.shapes[src][1]
    rng = np.random.default_rng([work.seed, layer, 16 + phase, 2])
    return rng.uniform(0.5, 1.5, k).astype(np.float32)


def single_gemv():
    """The small single-GEMV case: M=1, K=256, N=512, seed 0, uniform trits
    drawn first, then x ~ N(0, 1); s_w = 0.02."""
    rng = np.random.default_rng(0)
    t = rng.integers(-1, 2, size=(512, 256), dtype=np.int8)
    x = rng.standard_normal(256, dtype=np.float32)[None, :]
    return t, np.float32(0.02), x
