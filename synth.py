"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage types
(fp16, bf16, uint8 codes).  It holds none of the coding, decoding or GEMV
arithmetic: both the oracle and the HIP path receive these arrays as inputs.

Workloads (shapes of Llama-3.1-8B and Llama-70B MLP matrices, the matrices the
Unweight write-up compresses, "Understanding BF16 weight structure"; code
histograms stand in for the concentrated GPTQ codes of LazyWeights, Fig. 2):

  q4_256x1024          256x1024, 4-bit codes q = clamp(rint(N(7.5, 1.8)), 0, 15)
  q4_up_14336x4096     14336x4096 (up/gate), same code law
  q4_down_4096x14336   4096x14336 (down), q = clamp(rint(Laplace(7.5, b=1.2)), 0, 15)
  bf16_up_14336x4096   14336x4096 bf16 weights W = bf16(N(0, 0.02)), bf16 activations
  q6_mlp_70b           gate 28672x8192, up 28672x8192, down 8192x28672, 6-bit
                       codes q = clamp(rint(N(31.5, 5)), 0, 63), run back to back

For the quantised workloads each 256-weight super-block (256 consecutive
weights of one row) carries fp16 d ~ U(0.005, 0.02) and m = 8 d (exact in
fp16); activations are fp16 N(0, 1), drawn as 16 rows so that batch b uses the
first b.

Seeds: each matrix has a seed s (1000, 2000, 3000, 4000 and 5000..5002 in the
order above) and draws from SeedSequence(s).spawn(3), the three children
feeding (codes or W), (scales), (x) in that order.
"""
from __future__ import annotations

import dataclasses
import numpy as np

SUPER = 256          # weights per super-block (one tile row)
XROWS = 16           # activation rows drawn per matrix (max batch)


@dataclasses.dataclass(frozen=True)
class Matrix:
    seed: int
    name: str
    kind: str        # "q4", "q6" or "bf16"
    rows: int
    cols: int
    law: str         # "normal", "laplace" or "bf16normal"
    mu: float
    scale: float


WORKLOADS = {
    "q4_256x1024": [Matrix(1000, "q4_256x1024", "q4", 256, 1024, "normal", 7.5, 1.8)],
    "q4_up_14336x4096": [Matrix(2000, "q4_up_14336x4096", "q4", 14336, 4096, "normal", 7.5, 1.8)],
    "q4_down_4096x14336": [Matrix(3000, "q4_down_4096x14336", "q4", 4096, 14336, "laplace", 7.5, 1.2)],
    "bf16_up_14336x4096": [Matrix(4000, "bf16_up_14336x4096", "bf16", 14336, 4096, "bf16normal", 0.0, 0.02)],
    "q6_mlp_70b": [Matrix(5000, "q6_gate_28672x8192", "q6", 28672, 8192, "normal", 31.5, 5.0),
                   Matrix(5001, "q6_up_28672x8192", "q6", 28672, 8192, "normal", 31.5, 5.0),
                   Matrix(5002, "q6_down_8192x28672", "q6", 8192, 28672, "normal", 31.5, 5.0)],
}

# batch sizes each workload is checked at
BATCHES = {"q4_256x1024": (1,), "q4_up_14336x4096": (1,), "q4_down_4096x14336": (1, 4, 16),
           "bf16_up_14336x4096": (1,), "q6_mlp_70b": (1,)}

SMALL = "q4_256x1024"
DEFAULT = "q4_up_14336x4096"


def _rngs(seed: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3)]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of float32 values to bf16, returned as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _codes(rng, law: str, mu: float, scale: float, rows: int, cols: int, qmax: int,
           chunk: int = 1 << 24) -> np.ndarray:
    """q = clamp(rint(mu + scale * Z), 0, qmax), Z standard normal or Laplace(0, 1).

    Drawn in float32, chunked so that a 235M-weight matrix does not need a
    float64 copy of itself.
    """
    n = rows * cols
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        if law == "normal":
            z = rng.standard_normal(e - s, dtype=np.float32)
        elif law == "laplace":
            z = rng.laplace(0.0, 1.0, e - s).astype(np.float32)
        else:
            raise ValueError(law)
        v = np.rint(np.float32(mu) + np.float32(scale) * z)
        np.clip(v, 0, qmax, out=v)
        out[s:e] = v.astype(np.uint8)
    return out.reshape(rows, cols)


def gen_q(mat: Matrix, rows: int | None = None, cols: int | None = None):
    """Quantised matrix: (codes uint8 [R][C], d fp16-bits [R][C/256],
    m fp16-bits [R][C/256], x fp16-bits [16][C]).

    ``rows``/``cols`` override the shape (same law and seeds) for reduced cases.
    """
    R = mat.rows if rows is None else rows
    C = mat.cols if cols is None else cols
    assert C % SUPER == 0
    qmax = 15 if mat.kind == "q4" else 63
    rc, rs, rx = _rngs(mat.seed)
    codes = _codes(rc, mat.law, mat.mu, mat.scale, R, C, qmax)
    d = rs.uniform(0.005, 0.02, size=(R, C // SUPER)).astype(np.float16)
    m = (d.astype(np.float32) * 8).astype(np.float16)   # exact: power-of-two scale
    x = rx.standard_normal((XROWS, C)).astype(np.float16)
    return codes, d.view(np.uint16), m.view(np.uint16), x.view(np.uint16)


def gen_bf16(mat: Matrix, rows: int | None = None, cols: int | None = None):
    """BF16 matrix: (W bf16-bits [R][C], x bf16-bits [16][C])."""
    R = mat.rows if rows is None else rows
    C = mat.cols if cols is None else cols
    rw, _, rx = _rngs(mat.seed)
    n = R * C
    w = np.empty(n, dtype=np.uint16)
    chunk = 1 << 24
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        z = rw.standard_normal(e - s, dtype=np.float32) * np.float32(mat.scale)
        w[s:e] = f32_to_bf16_bits(z)
    x = f32_to_bf16_bits(rx.standard_normal((XROWS, C)).astype(np.float32))
    return w.reshape(R, C), x


def gen_q_custom(rows: int, cols: int, seed: int, qmax: int = 15, law: str = "normal",
                 mu: float = 7.5, scale: float = 1.8):
    """Same recipe as gen_q with an arbitrary seed and law (test cases)."""
    rc, rs, rx = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3)]
    if law == "uniform":
        codes = rc.integers(0, qmax + 1, size=(rows, cols), dtype=np.uint8)
    elif law == "const":
        codes = np.full((rows, cols), int(mu), dtype=np.uint8)
    else:
        codes = _codes(rc, law, mu, scale, rows, cols, qmax)
    d = rs.uniform(0.005, 0.02, size=(rows, cols // SUPER)).astype(np.float16)
    m = (d.astype(np.float32) * 8).astype(np.float16)
    x = rx.standard_normal((XROWS, cols)).astype(np.float16)
    return codes, d.view(np.uint16), m.view(np.uint16), x.view(np.uint16)


def gen_bf16_custom(rows: int, cols: int, seed: int, sigma: float = 0.02,
                    outlier_frac: float = 0.0):
    """bf16 N(0, sigma) weights; ``outlier_frac`` of them are scaled by 2^20 or
    2^-20 so that their exponents fall outside any 16-entry palette."""
    rw, ro, rx = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3)]
    z = rw.standard_normal(rows * cols, dtype=np.float32) * np.float32(sigma)
    if outlier_frac > 0:
        k = int(round(outlier_frac * z.size))
        idx = ro.choice(z.size, size=k, replace=False)
        sc = np.where(ro.random(k) < 0.5, np.float32(2.0 ** 20), np.float32(2.0 ** -20))
        z[idx] *= sc
    w = f32_to_bf16_bits(z).reshape(rows, cols)
    x = f32_to_bf16_bits(rx.standard_normal((XROWS, cols)).astype(np.float32))
    return w, x


def gen_fixed(rows: int, cols: int, bits: int, seed: int):
    """b-bit codes for the fixed-width paths: q = clamp(rint(N((2^b - 1)/2,
    2^b / 8.9)), 0, 2^b - 1) (the 4-bit law N(7.5, 1.8) scaled to b bits),
    fp16 d ~ U(0.005, 0.02) per 256 columns, m = 2^(b-1) d, fp16 x ~ N(0, 1)."""
    top = (1 << bits) - 1
    rc, rs, rx = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3)]
    codes = _codes(rc, "normal", top / 2.0, (1 << bits) / 8.9, rows, cols, top)
    d = rs.uniform(0.005, 0.02, size=(rows, cols // SUPER)).astype(np.float16)
    m = (d.astype(np.float32) * (1 << (bits - 1))).astype(np.float16)
    x = rx.standard_normal((XROWS, cols)).astype(np.float16)
    return codes, d.view(np.uint16), m.view(np.uint16), x.view(np.uint16)


def active_tiles(n_tiles: int, n_active: int, seed: int) -> np.ndarray:
    """A seeded set of n_active distinct tile indices in increasing order (the
    synthetic stand-in for a sparsity predictor's launch list)."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n_tiles, size=n_active, replace=False)).astype(np.int32)
