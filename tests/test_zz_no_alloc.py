"""GPU: lw_gemv_noalloc (lw_gemv with the split-column reduction's scratch in
the library's per-device array instead of the bundle's workspace) against
lw_gemv, through the C ABI, on two calls in a row, the second with a smaller
input: the same kernels and summation order, so the outputs are bit-identical,
and both are within the 1e-3 bar of the oracle."""
import numpy as np
import pytest

import oracle as O
import synth
from support import rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as T
    assert T.cuda.is_available(), "GPU tests need a GPU"
    return T


@pytest.fixture(scope="module")
def dg():
    import decode_gemv_amd as D
    return D


def _case(torch, dg, rows, cols, seed, batch, kind="q4"):
    qmax, mu, sc = (15, 7.5, 1.8) if kind == "q4" else (63, 31.5, 5.0)
    codes, d, m, x = synth.gen_q_custom(rows, cols, seed, qmax=qmax, mu=mu, scale=sc)
    k = dg.LW_Q4_PAIR if kind == "q4" else dg.LW_Q6_SINGLE
    b = dg.lw_bundle_build_q(k, codes, d, m)
    info = dg.lw_bundle_get_info(b)
    db = dg.upload(b)
    xt = torch.from_numpy(np.ascontiguousarray(x[:batch]).view(np.int16)).cuda()
    return codes, d, m, x, db, xt, info


@pytest.mark.parametrize("batch", [1, 3, 16])
def test_noalloc_equals_gemv_two_calls(torch, dg, batch):
    # first call: 192 x 14336 (56 column blocks: a split-column reduction across
    # workgroups), then a smaller input, 128 x 3584 (14 column blocks)
    for rows, cols, seed in ((192, 14336, 41), (128, 3584, 42)):
        print("noalloc", rows, cols, batch, flush=True)
        codes, d, m, x, db, xt, info = _case(torch, dg, rows, cols, seed, batch)
        y0 = torch.full((batch, rows), float("nan"), device="cuda")
        y1 = torch.full((batch, rows), float("nan"), device="cuda")
        dg.lw_gemv(db, xt, y0, batch)
        dg.lw_gemv_noalloc(db, xt, y1, batch)
        torch.cuda.synchronize()
        a, b = y0.cpu().numpy(), y1.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert rel_err(b, O.gemv_q(codes, d, m, x, batch)) <= 1e-3


def test_noalloc_repeated_and_6bit(torch, dg):
    # the array keeps the last call's contents: repeated calls on one stream
    # (and a 6-bit bundle with more row bands) still give lw_gemv's bits
    codes, d, m, x, db, xt, info = _case(torch, dg, 320, 7168, 43, 1, kind="q6")
    y0 = torch.full((1, 320), float("nan"), device="cuda")
    dg.lw_gemv(db, xt, y0, 1)
    for r in range(3):
        y1 = torch.full((1, 320), float("nan"), device="cuda")
        dg.lw_gemv_noalloc(db, xt, y1, 1)
        torch.cuda.synchronize()
        assert np.array_equal(y0.cpu().numpy().view(np.uint32), y1.cpu().numpy().view(np.uint32)), r
    assert rel_err(y0.cpu().numpy(), O.gemv_q(codes, d, m, x, 1)) <= 1e-3


def test_noalloc_refuses_oversized_reduction(torch, dg):
    # 4800 x 57344: 224 column blocks, 56 groups, 55 pair slots x 16 x 4800 rows
    # x 4 B = 16.9 MB, more than the 16 MiB array: refused before any launch
    rows, cols = 4800, 57344
    codes = np.full((rows, cols), 8, np.uint8)
    d = np.full((rows, cols // 256), 0x2000, np.uint16)
    b = dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, d)
    info = dg.lw_bundle_get_info(b)
    assert info["region_bytes"][dg.LW_REG_WORK] > 16 << 20
    db = dg.upload(b)
    xt = torch.zeros((1, cols), dtype=torch.int16, device="cuda")
    y = torch.zeros((1, rows), device="cuda")
    with pytest.raises(dg.LwError) as e:
        dg.lw_gemv_noalloc(db, xt, y, 1)
    assert e.value.status == dg.LW_E_UNSUPPORTED
