"""GPU tests of the exponent-only, palette and direct-palette pipelines of
"Unweight" ("Four approaches to using compressed weights", "How
reconstructive matmul works"): the transcode kernel's compact forms are
compared word for word with the oracle's, and the reconstructive
matrix-core GEMM with the oracle's fp64 GEMV over the exact bf16 weights
(max relative error 1e-3 with a floor of 0.01 rms, the S15 measure of
test_gpu_parity), in every variant, on shapes with a ragged last row block
and with verbatim segments."""
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
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits(rng.standard_normal((batch, cols), dtype=np.float32))


def dev(torch, a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype.itemsize == 2 else a.view(np.int32)).cuda()


def setup(dg, torch, rows, cols, seed, frac):
    w, _ = synth.gen_bf16_custom(rows, cols, seed, outlier_frac=frac)
    db = dg.upload(dg.lw_bundle_build_bf16(w))
    return w, db


def transcode(dg, torch, db, form, rows, cols):
    nt = (rows // 64) * (cols // 256)
    out = torch.zeros(rows * cols // (8 if form == dg.LW_FORM_PALETTE else 4), dtype=torch.int32, device="cuda")
    vr = torch.zeros(nt * 256, dtype=torch.int32, device="cuda")
    dg.lw_bf16_transcode(db, form, out, vr)
    return out, vr


SHAPES = [(64, 256, 0.0, 401), (192, 768, 0.004, 402), (320, 2304, 0.002, 403)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_transcode_matches_oracle(torch, dg, shape):
    rows, cols, frac, seed = shape
    say("transcode", shape)
    w, db = setup(dg, torch, rows, cols, seed, frac)
    ref = O.transcode_forms(O.build_bundle_bf16(w), w)
    for form, key in ((dg.LW_FORM_PALETTE, "palette"), (dg.LW_FORM_EXPONENT, "exponent")):
        out, vr = transcode(dg, torch, db, form, rows, cols)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref[key]), key
        assert np.array_equal(vr.cpu().numpy(), ref["vrank"]), key


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("batch", [1, 7, 16, 33, 64, 130])
def test_recon_gemm_matches_oracle(torch, dg, shape, batch):
    rows, cols, frac, seed = shape
    say("recon", shape, batch)
    w, db = setup(dg, torch, rows, cols, seed, frac)
    x = big_x(cols, batch, seed + 7)
    xd = dev(torch, x)
    ref = O.gemv_bf16(w, x, batch)
    work = torch.empty(8 * batch * rows * 4, dtype=torch.uint8, device="cuda")     # room for an 8-way column split
    for form in (dg.LW_FORM_PALETTE, dg.LW_FORM_EXPONENT):
        src, vr = transcode(dg, torch, db, form, rows, cols)
        for variant in range(-1, dg.LW_RECON_VARIANTS):
            for wk in (None, work):
                y = torch.full((batch, rows), float("nan"), device="cuda")
                dg.lw_recon_gemm(db, form, src, vr, xd, y, batch, variant, wk)
                torch.cuda.synchronize()
                yy = y.cpu().numpy()
                assert np.all(np.isfinite(yy)), (form, variant, wk is None)
                assert rel_err(yy, ref) <= TOL, (form, variant, wk is None, rel_err(yy, ref))


def test_recon_unit_vectors_give_columns(torch, dg):
    """x = e_c returns column c of W exactly (one product per output, fp32
    accumulation of zeros), verbatim segments included."""
    rows, cols = 128, 512
    w, db = setup(dg, torch, rows, cols, 411, 0.01)
    cs = [0, 63, 64, 300, 511]
    x = np.zeros((len(cs), cols), np.uint16)
    for i, c in enumerate(cs):
        x[i, c] = 0x3F80                                   # bf16 1.0
    wf = (w.astype(np.uint32) << 16).view(np.float32)
    for form in (dg.LW_FORM_PALETTE, dg.LW_FORM_EXPONENT):
        src, vr = transcode(dg, torch, db, form, rows, cols)
        y = torch.empty((len(cs), rows), device="cuda")
        dg.lw_recon_gemm(db, form, src, vr, dev(torch, x), y, len(cs), 2)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), wf[:, cs].T)


def test_recon_deterministic(torch, dg):
    rows, cols = 192, 1024
    w, db = setup(dg, torch, rows, cols, 421, 0.002)
    x = dev(torch, big_x(cols, 40, 422))
    src, vr = transcode(dg, torch, db, dg.LW_FORM_PALETTE, rows, cols)
    work = torch.empty(8 * 40 * rows * 4, dtype=torch.uint8, device="cuda")
    for variant, wk in ((3, None), (1, work)):            # unsplit, and split four ways (4 column blocks)
        ys = []
        for _ in range(2):
            y = torch.empty((40, rows), device="cuda")
            dg.lw_recon_gemm(db, dg.LW_FORM_PALETTE, src, vr, x, y, 40, variant, wk)
            torch.cuda.synchronize()
            ys.append(y.cpu().numpy())
        assert np.array_equal(ys[0], ys[1])


def test_recon_corrupt_ranks_stay_in_bounds(torch, dg):
    """Rank tables with entries past the store (or naming another row band's
    segments) must not send the kernel outside the store or the staged run:
    entries past the store are ignored, others only change values."""
    rows, cols = 192, 768
    w, db = setup(dg, torch, rows, cols, 451, 0.002)
    nv = dg.lw_bundle_get_info(dg.lw_bundle_build_bf16(w))["n_verbatim"]
    x = dev(torch, big_x(cols, 20, 452))
    src, vr = transcode(dg, torch, db, dg.LW_FORM_PALETTE, rows, cols)
    bad = np.random.default_rng(453).integers(-5, nv + 10 ** 6, size=vr.numel(), dtype=np.int64).astype(np.int32)
    for variant in (0, 3):
        y = torch.empty((20, rows), device="cuda")
        dg.lw_recon_gemm(db, dg.LW_FORM_PALETTE, src, dev(torch, bad), x, y, 20, variant)
        torch.cuda.synchronize()
        assert np.all(np.isfinite(y.cpu().numpy()))


def test_pipelines_through_the_table(torch, dg):
    """lw_gemm runs the pipeline (and variant) the table names; the direct
    palette pipeline needs an attached palette form; every pipeline agrees
    with the oracle."""
    rows, cols, batch = 192, 1280, 48
    w, db = setup(dg, torch, rows, cols, 431, 0.003)
    x = big_x(cols, batch, 432)
    xd = dev(torch, x)
    ref = O.gemv_bf16(w, x, batch)
    scratch = max(dg.lw_pipeline_scratch_bytes(db, p) for p in range(dg.LW_PIPE_COUNT))
    assert dg.lw_pipeline_scratch_bytes(db, dg.LW_PIPE_PALETTE) >= rows * cols // 2
    wbuf = torch.empty(scratch, dtype=torch.uint8, device="cuda")
    with pytest.raises(dg.LwError) as e:
        dg.lw_pipeline_set(db, 33, 64, dg.LW_PIPE_DIRECT_PALETTE)
    assert e.value.status == dg.LW_E_UNSUPPORTED
    pbuf = torch.empty(dg.lw_pipeline_scratch_bytes(db, dg.LW_PIPE_DIRECT_PALETTE), dtype=torch.uint8, device="cuda")
    dg.lw_bundle_attach_palette(db, pbuf)
    outs = {}
    for p in (dg.LW_PIPE_FULL_DECODE, dg.LW_PIPE_EXPONENT, dg.LW_PIPE_PALETTE, dg.LW_PIPE_DIRECT_PALETTE):
        dg.lw_pipeline_set(db, 33, 64, p)
        assert dg.lw_pipeline_get(db, batch) == p
        y = torch.full((batch, rows), float("nan"), device="cuda")
        dg.lw_gemm(db, xd, y, batch, wbuf)
        torch.cuda.synchronize()
        outs[p] = y.cpu().numpy()
        assert rel_err(outs[p], ref) <= TOL, p
    # the palette pipelines differ only in when the transcode runs
    assert np.array_equal(outs[dg.LW_PIPE_PALETTE], outs[dg.LW_PIPE_DIRECT_PALETTE])


def test_autotune_covers_the_reconstructive_pipelines(torch, dg):
    rows, cols = 320, 2304
    w, db = setup(dg, torch, rows, cols, 441, 0.002)
    x = dev(torch, big_x(cols, 256, 442))
    y = torch.empty((256, rows), device="cuda")
    scratch = max(dg.lw_pipeline_scratch_bytes(db, p) for p in range(dg.LW_PIPE_COUNT))
    wbuf = torch.empty(scratch, dtype=torch.uint8, device="cuda")
    pbuf = torch.empty(dg.lw_pipeline_scratch_bytes(db, dg.LW_PIPE_DIRECT_PALETTE), dtype=torch.uint8, device="cuda")
    dg.lw_bundle_attach_palette(db, pbuf)
    batches = [1, 16, 64, 256]
    us = dg.lw_autotune(db, batches, x, y, wbuf, reps=2)
    say("autotune us", us.tolist())
    for i, b in enumerate(batches):
        for p in (dg.LW_PIPE_FULL_DECODE, dg.LW_PIPE_EXPONENT, dg.LW_PIPE_PALETTE, dg.LW_PIPE_DIRECT_PALETTE):
            assert us[i, p] > 0
        best = int(np.argmax(np.where(us[i] > 0, -us[i], -np.inf)))
        assert dg.lw_pipeline_get(db, b) == best


@pytest.mark.parametrize("batch", [64, 256])
def test_recon_full_size(torch, dg, batch):
    mat = synth.WORKLOADS["bf16_up_14336x4096"][0]
    say("recon full size", batch)
    w, _ = synth.gen_bf16(mat)
    db = dg.upload(dg.lw_bundle_build_bf16(w))
    x = big_x(mat.cols, batch, 9)
    src, vr = transcode(dg, torch, db, dg.LW_FORM_PALETTE, mat.rows, mat.cols)
    y = torch.empty((batch, mat.rows), device="cuda")
    work = torch.empty(8 * batch * mat.rows * 4, dtype=torch.uint8, device="cuda")
    dg.lw_recon_gemm(db, dg.LW_FORM_PALETTE, src, vr, dev(torch, x), y, batch, -1, work)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(10).choice(mat.rows, 48, replace=False))
    assert rel_err(y.cpu().numpy()[:, rows], O.gemv_bf16(w, x, batch, rows=rows)) <= TOL


def test_recon_argument_errors(torch, dg):
    rows, cols = 64, 256
    w, db = setup(dg, torch, rows, cols, 461, 0.0)
    src, vr = transcode(dg, torch, db, dg.LW_FORM_PALETTE, rows, cols)
    x = dev(torch, big_x(cols, 4, 462))
    y = torch.empty((4, rows), device="cuda")
    for kw, status in ((dict(variant=dg.LW_RECON_VARIANTS), dg.LW_E_ARG), (dict(variant=-2), dg.LW_E_ARG)):
        with pytest.raises(dg.LwError) as e:
            dg.lw_recon_gemm(db, dg.LW_FORM_PALETTE, src, vr, x, y, 4, **kw)
        assert e.value.status == status
    with pytest.raises(dg.LwError) as e:                 # the exponent form is twice the palette form's size
        dg.lw_recon_gemm(db, dg.LW_FORM_EXPONENT, src, vr, x, y, 4)
    assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:
        dg.lw_recon_gemm(db, 7, src, vr, x, y, 4)
    assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:
        dg.lw_recon_gemm(db, dg.LW_FORM_PALETTE, src, vr, x, y, 0)
    assert e.value.status == dg.LW_E_ARG
    codes, d, m, _ = synth.gen_q_custom(64, 256, 463)
    qdb = dg.upload(dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m))
    with pytest.raises(dg.LwError) as e:
        dg.lw_bf16_transcode(qdb, dg.LW_FORM_PALETTE, src, vr)
    assert e.value.status == dg.LW_E_UNSUPPORTED
    with pytest.raises(dg.LwError) as e:                 # no palette form attached yet
        dg.lw_pipeline_set(db, 1, 1, dg.LW_PIPE_DIRECT_PALETTE)
    assert e.value.status == dg.LW_E_UNSUPPORTED
    assert dg.lw_pipeline_scratch_bytes(qdb, dg.LW_PIPE_PALETTE) == 0
