"""Helpers shared by the tests: the oracle over whole matrices on every host
core, and random complete prefix codes.

The oracle's C routines release Python's lock, and the rows of a GEMV are
independent, so splitting the rows into bands and running the unchanged
oracle on each band in a thread pool gives exactly the one-thread result in
a fraction of the time.  Nothing here computes anything the oracle does not.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle as O


def host_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


def _bands(rows: int, parts: int):
    cuts = [rows * i // parts for i in range(parts + 1)]
    return [np.arange(cuts[i], cuts[i + 1], dtype=np.int64) for i in range(parts) if cuts[i + 1] > cuts[i]]


def gemv_q_all(codes, d, m, x, batch: int) -> np.ndarray:
    """The oracle's fp64 GEMV on every row of a quantised matrix."""
    rows = codes.shape[0]
    n = host_threads()
    bands = _bands(rows, 4 * n)
    with ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(lambda r: O.gemv_q(codes, d, m, x, batch, rows=r), bands))
    return np.concatenate(parts, axis=1)


def gemv_bf16_all(w, x, batch: int) -> np.ndarray:
    """The oracle's fp64 GEMV on every row of a bf16 matrix."""
    rows = w.shape[0]
    n = host_threads()
    bands = _bands(rows, 4 * n)
    with ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(lambda r: O.gemv_bf16(w, x, batch, rows=r), bands))
    return np.concatenate(parts, axis=1)


def mlp_pass_all(gate, up, down, x, batch: int):
    """The oracle's SwiGLU pass (O.mlp_pass_q's steps) with each GEMV over
    row bands: returns (g, u, h bits, y)."""
    g = gemv_q_all(*gate, x, batch)
    u = gemv_q_all(*up, x, batch)
    h = O.swiglu(g, u)
    return g, u, h, gemv_q_all(*down, h, batch)


def activation_spread(down, h_bits, h_ref_bits, chunk: int = 1024) -> np.ndarray:
    """sum_j |w_ij| |h_j - h_ref_j| for every output i of the down matrix
    (codes, d, m) and batch row: how far apart two fp16 activation vectors
    can move its GEMV.  With w = d*q - m per 256-weight block (fp64)."""
    codes, d, m = down
    hd = np.abs(np.asarray(h_bits, np.uint16).view(np.float16).astype(np.float64) -
                np.asarray(h_ref_bits, np.uint16).view(np.float16).astype(np.float64))
    rows = codes.shape[0]
    out = np.zeros((hd.shape[0], rows))
    for r0 in range(0, rows, chunk):
        q = codes[r0:r0 + chunk].astype(np.float64)
        ds = np.repeat(np.asarray(d[r0:r0 + chunk], np.uint16).view(np.float16).astype(np.float64), 256, axis=1)
        ms = np.repeat(np.asarray(m[r0:r0 + chunk], np.uint16).view(np.float16).astype(np.float64), 256, axis=1)
        out[:, r0:r0 + chunk] = hd @ np.abs(ds * q - ms).T
    return out


def pass_within(y, yref, spread, tol: float) -> bool:
    """|y - yref| <= tol * max(|yref|, 0.01 rms(yref)) + spread on every
    output: the usual bar plus what the activations' fp16 rounding
    differences carry through the down GEMV."""
    ref = np.asarray(yref, np.float64)
    floor = 0.01 * np.sqrt(np.mean(ref ** 2))
    err = np.abs(np.asarray(y, np.float64) - ref)
    return bool(np.all(err <= tol * np.maximum(np.abs(ref), floor) + spread * (1 + 1e-9)))


def rel_err(y, ref) -> float:
    """max |y - ref| / max(|ref|, 0.01 rms(ref)) over all outputs."""
    ref = np.asarray(ref, np.float64)
    floor = 0.01 * np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref) / np.maximum(np.abs(ref), floor)))


def random_complete_lengths(rng, n_alpha: int, n_sym: int, max_depth: int = 11):
    """Lengths of a random complete prefix code over n_sym of n_alpha symbols:
    split random leaves of a binary tree (depth <= max_depth) until n_sym
    leaves exist.  Returns (lengths u8 [n_alpha], the coded symbols)."""
    leaves = [0]
    while len(leaves) < n_sym:
        cand = [i for i, dpt in enumerate(leaves) if dpt < max_depth]
        i = cand[rng.integers(len(cand))]
        dpt = leaves.pop(i)
        leaves += [dpt + 1, dpt + 1]
    syms = rng.permutation(n_alpha)[:n_sym]
    lens = np.zeros(n_alpha, np.uint8)
    lens[syms] = leaves
    return lens, syms


def codes_over(rng, pairs: bool, syms, rows: int = 64, cols: int = 256) -> np.ndarray:
    """A code matrix in which exactly the given symbols occur (pair symbols
    lo | hi << 4 of adjacent columns when `pairs`)."""
    n = rows * cols // (2 if pairs else 1)
    pick = np.concatenate([syms, rng.choice(syms, n - len(syms))])
    rng.shuffle(pick)
    if pairs:
        q = np.empty(rows * cols, np.uint8)
        q[0::2] = pick & 15
        q[1::2] = pick >> 4
    else:
        q = pick.astype(np.uint8)
    return q.reshape(rows, cols)


def plan_of(bundle):
    """The comparison plan a bundle carries in its derived GPU tables
    (lw_gputab.plan), as a dict of its fields."""
    import decode_gemv_amd as dg
    g = dg.lw_bundle_region(bundle, dg.LW_REG_GPUTAB, np.uint32)
    off = (16 * 3 + 256 * 3)                 # limlj, len, base, payload, payload_hi, symval
    w = g[off:off + 24]
    return dict(plan=int(w[0]), sad_k=int(w[1]), c8=[int(w[2]), int(w[3])], c8m1=[int(w[4]), int(w[5])],
                c16=int(w[6]), c16m1=int(w[7]), xsel=[int(w[8]), int(w[9])], xk=[int(w[10]), int(w[11])],
                lut_lo=int(w[12]), lut_hi=int(w[13]), cbase=[int(np.int32(v)) for v in w[14:18]],
                ncmp=int(w[18]))
