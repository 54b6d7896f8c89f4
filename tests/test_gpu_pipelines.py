"""GPU tests of the execution pipelines of "Unweight" ("Four approaches to
using compressed weights"): full decode + library GEMM against the oracle's
fp64 GEMV over the exact bf16 weights, the per-bundle pipeline table behind
lw_gemm, and the autotuner that fills it.  Tolerance: the S15 measure of
test_gpu_parity (max relative error 1e-3 with a floor of 0.01 rms)."""
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


def big_x(cols, batch, seed):
    """bf16 activations [batch][cols], N(0, 1), seeded (batches beyond synth's 16 rows)."""
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits(rng.standard_normal((batch, cols), dtype=np.float32))


def setup(dg, torch, rows, cols, seed, frac=0.0):
    w, _ = synth.gen_bf16_custom(rows, cols, seed, outlier_frac=frac)
    db = dg.upload(dg.lw_bundle_build_bf16(w))
    wbuf = torch.empty(rows * cols, dtype=torch.int16, device="cuda")
    return w, db, wbuf


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


@pytest.mark.parametrize("case", [(64, 256, 0.0, 301), (192, 1280, 0.01, 302), (320, 2304, 0.002, 303)],
                         ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("batch", [1, 5, 16, 33, 300])
def test_full_decode_matches_oracle(torch, dg, case, batch):
    rows, cols, frac, seed = case
    say("full decode", case, batch)
    w, db, wbuf = setup(dg, torch, rows, cols, seed, frac)
    x = big_x(cols, batch, seed + 1)
    y = torch.full((batch, rows), float("nan"), device="cuda")
    dg.lw_gemm_full_decode(db, wbuf, dev(torch, x), y, batch)
    torch.cuda.synchronize()
    assert np.array_equal(wbuf.cpu().numpy().view(np.uint16).reshape(rows, cols), w)   # the decoded weights
    assert rel_err(y.cpu().numpy(), O.gemv_bf16(w, x, batch)) <= TOL


def test_full_decode_full_size_batch64(torch, dg):
    mat = synth.WORKLOADS["bf16_up_14336x4096"][0]
    say("full decode full size", mat.name)
    w, _ = synth.gen_bf16(mat)
    db = dg.upload(dg.lw_bundle_build_bf16(w))
    wbuf = torch.empty(mat.rows * mat.cols, dtype=torch.int16, device="cuda")
    x = big_x(mat.cols, 64, 7)
    y = torch.empty((64, mat.rows), device="cuda")
    dg.lw_gemm_full_decode(db, wbuf, dev(torch, x), y, 64)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(8).choice(mat.rows, 48, replace=False))
    assert rel_err(y.cpu().numpy()[:, rows], O.gemv_bf16(w, x, 64, rows=rows)) <= TOL


def test_gemm_follows_the_table(torch, dg):
    rows, cols = 192, 1280
    w, db, wbuf = setup(dg, torch, rows, cols, 311)
    x = big_x(cols, 64, 312)
    xd = dev(torch, x)
    out = {}
    for name, batch, fn in (("fused8", 8, lambda y: dg.lw_gemv(db, xd, y, 8)),
                            ("full8", 8, lambda y: dg.lw_gemm_full_decode(db, wbuf, xd, y, 8)),
                            ("full64", 64, lambda y: dg.lw_gemm_full_decode(db, wbuf, xd, y, 64))):
        y = torch.empty((batch, rows), device="cuda")
        fn(y)
        torch.cuda.synchronize()
        out[name] = y.cpu().numpy()
    # default table: fused up to 16, full decode beyond
    assert dg.lw_pipeline_get(db, 8) == dg.LW_PIPE_FUSED and dg.lw_pipeline_get(db, 64) == dg.LW_PIPE_FULL_DECODE
    y = torch.empty((8, rows), device="cuda")
    dg.lw_gemm(db, xd, y, 8, wbuf)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), out["fused8"])
    y = torch.empty((64, rows), device="cuda")
    dg.lw_gemm(db, xd, y, 64, wbuf)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), out["full64"])
    dg.lw_pipeline_set(db, 5, 8, dg.LW_PIPE_FULL_DECODE)          # buckets (4, 8]: full decode
    assert dg.lw_pipeline_get(db, 8) == dg.LW_PIPE_FULL_DECODE and dg.lw_pipeline_get(db, 4) == dg.LW_PIPE_FUSED
    y = torch.empty((8, rows), device="cuda")
    dg.lw_gemm(db, xd, y, 8, wbuf)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), out["full8"])
    with pytest.raises(dg.LwError) as e:
        dg.lw_pipeline_set(db, 20, 40, dg.LW_PIPE_FUSED)          # the fused kernels stop at 16
    assert e.value.status == dg.LW_E_UNSUPPORTED


def test_autotune_sets_the_fastest(torch, dg):
    rows, cols = 320, 2304
    w, db, wbuf = setup(dg, torch, rows, cols, 321)
    batches = [1, 8, 16, 64, 256]
    x = dev(torch, big_x(cols, 256, 322))
    y = torch.empty((256, rows), device="cuda")
    us = dg.lw_autotune(db, batches, x, y, wbuf, reps=3)
    say("autotune us", us.tolist())
    for i, b in enumerate(batches):
        if b <= 16:
            assert us[i, dg.LW_PIPE_FUSED] > 0
        else:
            assert us[i, dg.LW_PIPE_FUSED] == -1
        assert us[i, dg.LW_PIPE_FULL_DECODE] > 0
        best = int(np.argmax(np.where(us[i] > 0, -us[i], -np.inf)))
        assert dg.lw_pipeline_get(db, b) == best


def test_quantised_bundles_have_no_full_decode(torch, dg):
    codes, d, m, x = synth.gen_q_custom(64, 512, 331)
    db = dg.upload(dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m))
    wbuf = torch.empty(64 * 512, dtype=torch.int16, device="cuda")
    y = torch.empty((32, 64), device="cuda")
    xd = dev(torch, np.zeros((32, 512), np.uint16))
    with pytest.raises(dg.LwError) as e:
        dg.lw_gemm_full_decode(db, wbuf, xd, y, 32)
    assert e.value.status == dg.LW_E_UNSUPPORTED
    with pytest.raises(dg.LwError) as e:
        dg.lw_gemm(db, xd, y, 32, wbuf)
    assert e.value.status == dg.LW_E_UNSUPPORTED
