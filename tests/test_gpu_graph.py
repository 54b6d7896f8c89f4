"""HIP graph capture of the C-ABI calls: a captured lw_gemv / lw_twin_gemv /
lw_decode_only must give, on every replay, exactly what the eager call gives.

The split-column reduction meets in pair slots of the bundle's workspace and
leaves them empty again inside the kernel (no memset node), so repeated
replays are the case under test.  Between replays the program does its own eager work
(other launches on the same bundle) and synchronises, as bench.py does.
"""
import numpy as np
import pytest

import oracle as O
import synth

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


def _replays_match(torch, launch, outs, n_replays=4, between=None):
    """Run `launch` eagerly, capture it, replay n times; every replay must
    reproduce the eager outputs bit for bit."""
    for o in outs:
        o.fill_(float("nan")) if o.is_floating_point() else o.zero_()
    launch()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    for r in range(n_replays):
        for o in outs:
            o.fill_(float("nan")) if o.is_floating_point() else o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"replay {r} differs from eager"
        if between is not None:
            between()
            torch.cuda.synchronize()


@pytest.mark.parametrize("rows,cols,batch", [(192, 1024, 1), (256, 4096, 3), (128, 2048, 16)])
def test_graph_gemv_q4(torch, dg, rows, cols, batch):
    print("graph gemv q4", rows, cols, batch, flush=True)
    codes, d, m, x = synth.gen_q_custom(rows, cols, 700 + batch)
    db = dg.upload(dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m))
    xt = torch.from_numpy(np.ascontiguousarray(x[:batch]).view(np.int16)).cuda()
    y = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y)
    _replays_match(torch, lambda: dg.lw_gemv(db, xt, y, batch), [y],
                   between=lambda: dg.lw_gemv(db, xt, y2, batch))
    ref = O.gemv_q(codes, d, m, x, batch)
    scale = np.maximum(np.abs(ref), 0.01 * np.sqrt(np.mean(ref ** 2)))
    assert np.max(np.abs(y.cpu().numpy() - ref) / scale) <= 1e-3


def test_graph_gemv_bf16(torch, dg):
    print("graph gemv bf16", flush=True)
    w, x = synth.gen_bf16_custom(128, 2048, 710, outlier_frac=1e-3)
    db = dg.upload(dg.lw_bundle_build_bf16(w))
    xt = torch.from_numpy(np.ascontiguousarray(x[:2]).view(np.int16)).cuda()
    y = torch.empty((2, 128), dtype=torch.float32, device="cuda")
    _replays_match(torch, lambda: dg.lw_gemv(db, xt, y, 2), [y])


def test_graph_twin_and_decode(torch, dg):
    print("graph twin and decode-only", flush=True)
    rows, cols = 128, 4096
    codes, d, m, x = synth.gen_q_custom(rows, cols, 720)
    db = dg.upload(dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m))
    twin, dmw = dg.lw_twin_build(codes, 4, d, m)
    tw = torch.from_numpy(twin).cuda()
    dmt = torch.from_numpy(dmw.view(np.int32)).cuda()
    xt = torch.from_numpy(np.ascontiguousarray(x[:1]).view(np.int16)).cuda()
    y = torch.empty((1, rows), dtype=torch.float32, device="cuda")
    _replays_match(torch, lambda: dg.lw_twin_gemv(tw, dmt, 4, rows, cols, xt, y, 1), [y])
    out = torch.zeros(rows * cols // 2, dtype=torch.uint8, device="cuda")
    _replays_match(torch, lambda: dg.lw_decode_only(db, out), [out])
    packed = out.cpu().numpy().reshape(rows, cols // 2)
    assert np.array_equal(packed & 15, codes[:, 0::2]) and np.array_equal(packed >> 4, codes[:, 1::2])
