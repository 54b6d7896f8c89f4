"""GPU parity of the tile-skipping fixed-width GEMV (lw_skip_gemv) against the
oracle's listed-tile GEMV ("Software-Defined Bandwidth Expansion", IV-C).

Rows of listed tiles must agree with the oracle's fp64 result within max
relative error 1e-3 (the S15 measure of test_gpu_parity); rows of every other
tile must keep what y held before the call (a NaN sentinel here).
"""
import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def torch():
    import torch as T
    assert T.cuda.is_available(), "GPU tests need a GPU"
    return T


@pytest.fixture(scope="module")
def dg():
    import decode_gemv_amd as D
    return D


def say(*a):
    print(*a, flush=True)


def rel_err(y, ref):
    ref = np.asarray(ref, np.float64)
    floor = 0.01 * np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref) / np.maximum(np.abs(ref), floor)))


def run_skip(dg, torch, words, dm, bits, rows, cols, tiles, x, batch):
    w_d = torch.from_numpy(words.view(np.int32)).cuda()
    dm_d = torch.from_numpy(dm.view(np.int32)).cuda()
    t_d = torch.from_numpy(np.ascontiguousarray(tiles, np.int32)).cuda()
    x_d = torch.from_numpy(np.ascontiguousarray(x[:batch]).view(np.int16)).cuda()
    y = torch.full((batch, rows), float("nan"), dtype=torch.float32, device="cuda")
    dg.lw_skip_gemv(w_d, dm_d, bits, rows, cols, t_d, x_d, y, batch)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(y, ref, rows, listed):
    act = np.zeros(rows // 64, bool)
    act[listed] = True
    rmask = np.repeat(act, 64)
    assert np.all(np.isnan(y[:, ~rmask])), "rows of unlisted tiles were written"
    if rmask.any():
        assert np.all(np.isfinite(y[:, rmask]))
        e = rel_err(y[:, rmask], ref[:, rmask])
        assert e <= TOL, e
        return e
    return 0.0


CASES = [
    # bits, rows, cols, seed: one tile, several tiles, chunk counts that leave
    # idle chunk lanes (n_jc not a multiple of 4), and long rows (several
    # chunks per thread)
    (4, 64, 256, 1), (4, 192, 768, 2), (2, 128, 1280, 3), (8, 128, 1280, 4), (2, 64, 256, 5),
    (8, 192, 2304, 6), (4, 128, 14336, 7), (2, 64, 8192, 8), (8, 64, 4096, 9),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}_{c[1]}x{c[2]}")
@pytest.mark.parametrize("batch", [1, 2, 3, 4])
def test_skip_all_tiles(torch, dg, case, batch):
    bits, rows, cols, seed = case
    say("skip all", bits, rows, cols, batch)
    codes, d, m, x = synth.gen_fixed(rows, cols, bits, seed)
    words, dm = dg.lw_skip_pack(codes, bits, d, m)
    tiles = np.arange(rows // 64, dtype=np.int32)
    y = run_skip(dg, torch, words, dm, bits, rows, cols, tiles, x, batch)
    ref = O.skip_gemv(words, dm, bits, rows, cols, tiles, x, batch)
    check(y, ref, rows, tiles)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_skip_listed_subset_duplicates_and_junk(torch, dg, bits):
    rows, cols = 64 * 10, 1024
    say("skip subset", bits)
    codes, d, m, x = synth.gen_fixed(rows, cols, bits, 20 + bits)
    words, dm = dg.lw_skip_pack(codes, bits, d, m)
    tiles = np.array([7, 2, 7, -1, 9, 10, 2, 123456, 0], np.int32)   # duplicates and entries naming no tile
    listed = [0, 2, 7, 9]
    for batch in (1, 4):
        y = run_skip(dg, torch, words, dm, bits, rows, cols, tiles, x, batch)
        ref = O.skip_gemv(words, dm, bits, rows, cols, tiles, x, batch)
        check(y, ref, rows, listed)
        y2 = run_skip(dg, torch, words, dm, bits, rows, cols, tiles, x, batch)
        assert np.array_equal(np.nan_to_num(y, nan=7.0), np.nan_to_num(y2, nan=7.0)), "not deterministic"


def test_skip_only_junk_and_empty_list(torch, dg):
    rows, cols, bits = 128, 512, 4
    codes, d, m, x = synth.gen_fixed(rows, cols, bits, 31)
    words, dm = dg.lw_skip_pack(codes, bits, d, m)
    y = run_skip(dg, torch, words, dm, bits, rows, cols, np.array([-5, 2, 99], np.int32), x, 1)
    assert np.all(np.isnan(y))
    y = run_skip(dg, torch, words, dm, bits, rows, cols, np.zeros(0, np.int32), x, 1)
    assert np.all(np.isnan(y))


def test_skip_zero_weights_and_unit_vector(torch, dg):
    """Codes equal to 2^(b-1) with m = 2^(b-1) d make every weight zero: the
    kernel's d * sum(q x) - m * sum(x) (two fp32 sums in different orders)
    must cancel to within 1e-6 of sum |m x|; x = e_c gives the dequantised
    column c (the oracle's special cases)."""
    rows, cols, bits = 128, 768, 4
    codes, d, m, x = synth.gen_fixed(rows, cols, bits, 33)
    words, dm = dg.lw_skip_pack(np.full_like(codes, 8), bits, d, m)
    y = run_skip(dg, torch, words, dm, bits, rows, cols, np.arange(2, dtype=np.int32), x, 2)
    mf = m.view(np.float16).astype(np.float64).repeat(256, axis=1)          # [rows][cols]
    scale = np.abs(x[:2].view(np.float16).astype(np.float64)) @ np.abs(mf).T   # [batch][rows]
    assert np.all(np.abs(y) <= 1e-6 * scale)
    words, dm = dg.lw_skip_pack(codes, bits, d, m)
    e = np.zeros((1, cols), np.float16)
    e[0, 300] = 1.0
    y = run_skip(dg, torch, words, dm, bits, rows, cols, np.arange(2, dtype=np.int32), e.view(np.uint16), 1)
    ref = O.skip_gemv(words, dm, bits, rows, cols, np.arange(2), e.view(np.uint16), 1)
    assert rel_err(y, ref) <= 1e-6


@pytest.mark.parametrize("shape", [("page", 1024, 4096, 2, 6), ("up", 14336, 4096, 4, None),
                                   ("up40", 14336, 4096, 4, 0.4)])
def test_skip_full_size(torch, dg, shape):
    """The page's worked configuration (1024 rows, K=4096, 2-bit codes, 6 of
    the 16 tiles active) and the 14336x4096 4-bit matrix, all tiles and a 40 % list;
    sampled listed rows against the oracle."""
    name, rows, cols, bits, act = shape
    say("skip full", name)
    codes, d, m, x = synth.gen_fixed(rows, cols, bits, 40)
    words, dm = dg.lw_skip_pack(codes, bits, d, m)
    nt = rows // 64
    if act is None:
        tiles = np.arange(nt, dtype=np.int32)
    else:
        n_act = act if isinstance(act, int) else int(round(act * nt))
        tiles = synth.active_tiles(nt, n_act, 41)
    y = run_skip(dg, torch, words, dm, bits, rows, cols, tiles, x, 1)
    sample = np.sort(np.random.default_rng(42).choice(tiles, size=min(len(tiles), 6), replace=False))
    ref = O.skip_gemv(words, dm, bits, rows, cols, sample, x, 1)
    rows_s = np.concatenate([np.arange(64 * t, 64 * t + 64) for t in sample])
    assert rel_err(y[:, rows_s], ref[:, rows_s]) <= TOL
    act_rows = np.repeat(np.isin(np.arange(nt), tiles), 64)
    assert np.all(np.isfinite(y[:, act_rows])) and np.all(np.isnan(y[:, ~act_rows]))
