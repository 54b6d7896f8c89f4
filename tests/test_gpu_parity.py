"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Decoded codes and bf16 weights must be bit-exact; GEMV outputs must agree with
the oracle's fp64 GEMV within max relative error 1e-3, where the relative
error of an output is |y - y_ref| / max(|y_ref|, 0.01 * rms(y_ref)) (the floor
keeps rows whose exact value is near zero from dividing by ~0; fp32
accumulation over <= 28672 terms is far inside this bound).
"""
import numpy as np
import pytest

import oracle as O
import synth
from support import codes_over, gemv_bf16_all, gemv_q_all, plan_of, random_complete_lengths

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


def rel_err(y, ref):
    ref = np.asarray(ref, np.float64)
    floor = 0.01 * np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref) / np.maximum(np.abs(ref), floor)))


def say(*a):
    print(*a, flush=True)


def _upload(dg, torch, b):
    return dg.upload(b)


def _run_gemv(dg, torch, db, x_bits, batch, rows):
    x = torch.from_numpy(np.ascontiguousarray(x_bits[:batch]).view(np.int16)).cuda()
    y = torch.full((batch, rows), float("nan"), dtype=torch.float32, device="cuda")
    dg.lw_gemv(db, x, y, batch)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _decode_q(dg, torch, db, kind, rows, cols, n_tiles):
    nbytes = rows * cols // 2 if kind == dg.LW_Q4_PAIR else rows * cols
    out = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    lb = torch.zeros(n_tiles * 32, dtype=torch.int32, device="cuda")
    dg.lw_decode_only(db, out, lane_bits=lb)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    if kind == dg.LW_Q4_PAIR:
        o = o.reshape(rows, cols // 2)
        q = np.empty((rows, cols), np.uint8)
        q[:, 0::2] = o & 15
        q[:, 1::2] = o >> 4
    else:
        q = o.reshape(rows, cols)
    return q, lb.cpu().numpy().view(np.uint32)


SMALL_Q = [
    # kind, rows, cols, law, seed  (edge shapes: one tile, odd row bands,
    # column blocks not a multiple of four, several column groups, whole-row
    # workgroups with all and with some wavefronts active, 14-wavefront
    # workgroups in two and three column groups)
    ("q4", 64, 256, "normal", 101), ("q4", 192, 768, "normal", 102), ("q4", 256, 1024, "normal", 103),
    ("q4", 128, 1280, "laplace", 104), ("q4", 320, 2304, "normal", 105), ("q4", 64, 4096, "normal", 106),
    ("q4", 192, 3584, "normal", 109), ("q6", 128, 3328, "normal", 115),
    ("q4", 128, 7168, "normal", 116), ("q4", 64, 10752, "laplace", 117), ("q6", 64, 7168, "normal", 118),
    ("q4", 128, 512, "uniform", 107), ("q4", 64, 512, "const", 108),
    ("q6", 64, 256, "normal", 111), ("q6", 192, 1280, "normal", 112), ("q6", 128, 2048, "uniform", 113),
    ("q6", 64, 768, "const", 114),
]


def _gen_small(kind, rows, cols, law, seed):
    if kind == "q4":
        return synth.gen_q_custom(rows, cols, seed, qmax=15, law=law, mu=7.5, scale=1.8)
    return synth.gen_q_custom(rows, cols, seed, qmax=63, law=law, mu=31.5, scale=5.0)


@pytest.mark.parametrize("case", SMALL_Q, ids=lambda c: "-".join(map(str, c)))
def test_decode_only_bit_exact_small(torch, dg, case):
    kind_s, rows, cols, law, seed = case
    say("decode", case)
    kind = dg.LW_Q4_PAIR if kind_s == "q4" else dg.LW_Q6_SINGLE
    codes, d, m, x = _gen_small(*case)
    b = dg.lw_bundle_build_q(kind, codes, d, m)
    info = dg.lw_bundle_get_info(b)
    db = _upload(dg, torch, b)
    q, bits = _decode_q(dg, torch, db, kind, rows, cols, info["n_tiles"])
    assert np.array_equal(q, codes)
    ob = O.build_bundle_q(kind, codes, d, m)
    _, obits = O.decode_bundle_q(ob)
    assert np.array_equal(bits, obits)


@pytest.mark.parametrize("case", SMALL_Q, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 7])
def test_gemv_small(torch, dg, case, batch):
    kind_s, rows, cols, law, seed = case
    say("gemv", case, batch)
    kind = dg.LW_Q4_PAIR if kind_s == "q4" else dg.LW_Q6_SINGLE
    codes, d, m, x = _gen_small(*case)
    b = dg.lw_bundle_build_q(kind, codes, d, m)
    db = _upload(dg, torch, b)
    y = _run_gemv(dg, torch, db, x, batch, rows)
    ref = O.gemv_q(codes, d, m, x, batch)
    assert rel_err(y, ref) <= TOL
    # deterministic: a second call gives identical bits
    y2 = _run_gemv(dg, torch, db, x, batch, rows)
    assert np.array_equal(y, y2)


def test_gemv_all_eights_is_zero(torch, dg):
    codes = np.full((128, 1024), 8, np.uint8)
    _, d, m, x = synth.gen_q_custom(128, 1024, 120)
    db = _upload(dg, torch, dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m))
    y = _run_gemv(dg, torch, db, x, 2, 128)
    assert np.all(np.abs(y) < 1e-6)


def test_twin_small(torch, dg):
    for rows, cols, seed in ((64, 256, 130), (192, 1024, 131), (128, 4096, 132), (64, 14336, 133)):
        codes, d, m, x = synth.gen_q_custom(rows, cols, seed)
        twin, dm = dg.lw_twin_build(codes, 4, d, m)
        tw = torch.from_numpy(twin).cuda()
        dmt = torch.from_numpy(dm.view(np.int32)).cuda()
        for batch in (1, 4, 16):
            say("twin", rows, cols, batch)
            xt = torch.from_numpy(np.ascontiguousarray(x[:batch]).view(np.int16)).cuda()
            y = torch.full((batch, rows), float("nan"), device="cuda")
            dg.lw_twin_gemv(tw, dmt, 4, rows, cols, xt, y, batch)
            torch.cuda.synchronize()
            assert rel_err(y.cpu().numpy(), O.gemv_q(codes, d, m, x, batch)) <= TOL


def test_argument_errors_device(torch, dg):
    codes, d, m, x = synth.gen_q_custom(64, 256, 140)
    b = dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_upload(b, small)
    assert e.value.status == dg.LW_E_ARG
    db = _upload(dg, torch, b)
    xt = torch.zeros((1, 256), dtype=torch.int16, device="cuda")
    y = torch.zeros((1, 64), device="cuda")
    with pytest.raises(dg.LwError) as e:
        dg.lw_gemv(db, xt, y, 17)
    assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:
        dg.lw_decode_only(db, torch.zeros(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == dg.LW_E_ARG


# ------------------------------------------------------------------ full sizes
# Every output row is compared with the oracle's fp64 GEMV (over row bands on
# every host core, the same numbers the one-thread oracle gives), in the
# launch configuration bench.py times (one lw_gemv call on the bundle).

@pytest.mark.parametrize("wl", ["q4_256x1024", "q4_up_14336x4096", "q4_down_4096x14336"])
def test_full_size_q4(torch, dg, wl):
    mat = synth.WORKLOADS[wl][0]
    say("full", mat.name)
    codes, d, m, x = synth.gen_q(mat)
    b = dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m)
    info = dg.lw_bundle_get_info(b)
    db = _upload(dg, torch, b)
    q, bits = _decode_q(dg, torch, db, dg.LW_Q4_PAIR, mat.rows, mat.cols, info["n_tiles"])
    assert np.array_equal(q, codes)
    del q
    _, obits = O.decode_bundle_q(O.build_bundle_q(O.Q4, codes, d, m))
    assert np.array_equal(bits, obits)
    for batch in synth.BATCHES[wl]:
        say("full gemv", mat.name, batch)
        y = _run_gemv(dg, torch, db, x, batch, mat.rows)
        assert rel_err(y, gemv_q_all(codes, d, m, x, batch)) <= TOL


_Q6 = {}


def _q6_matrix(i):
    """Inputs of 70B MLP matrix i (gate, up, down), generated once per session."""
    if i not in _Q6:
        _Q6[i] = synth.gen_q(synth.WORKLOADS["q6_mlp_70b"][i])
    return _Q6[i]


@pytest.mark.parametrize("i", [0, 1, 2], ids=["gate", "up", "down"])
def test_full_size_q6(torch, dg, i):
    """Each 70B MLP matrix (gate and up 28672x8192, down 8192x28672): decode
    bit-exact and every GEMV row against the oracle, at batch 1 and at batch
    16 (the matrix-core kernel, whose column groups -- 8 for gate and up, 28
    for down -- meet in a three- or five-level exchange tree)."""
    mat = synth.WORKLOADS["q6_mlp_70b"][i]
    say("full", mat.name)
    codes, d, m, x = _q6_matrix(i)
    b = dg.lw_bundle_build_q(dg.LW_Q6_SINGLE, codes, d, m)
    info = dg.lw_bundle_get_info(b)
    db = _upload(dg, torch, b)
    q, _ = _decode_q(dg, torch, db, dg.LW_Q6_SINGLE, mat.rows, mat.cols, info["n_tiles"])
    assert np.array_equal(q, codes)
    del q
    for batch in (1, 16):
        say("full gemv", mat.name, batch)
        y = _run_gemv(dg, torch, db, x, batch, mat.rows)
        assert rel_err(y, gemv_q_all(codes, d, m, x, batch)) <= TOL


def test_full_size_mlp_pass_70b(torch, dg):
    """The chained 70B pass at full shape: gate and up on x, lw_swiglu to fp16
    h, down on h, all on one stream.  g and u match the oracle's GEMVs, h is
    within one fp16 ulp of the oracle's SwiGLU of the GPU's own g and u (the
    fp32 sums are within 1e-3, but a gate output near zero carries a large
    relative error into silu, so h is compared on the same inputs), and y
    matches the oracle's down GEMV of that h, and the oracle's whole fp64
    pass within 1e-3 plus the down GEMV of the two passes' activation
    differences (sum_j |w_ij| |h_j - h_ref_j|)."""
    say("full mlp pass 70b")
    from support import mlp_pass_all
    mats = [_q6_matrix(i) for i in range(3)]
    dbs = [_upload(dg, torch, dg.lw_bundle_build_q(dg.LW_Q6_SINGLE, *mm[:3])) for mm in mats]
    x = mats[0][3]
    R, C = mats[0][0].shape
    xt = torch.from_numpy(np.ascontiguousarray(x[:1]).view(np.int16)).cuda()
    g = torch.empty((1, R), dtype=torch.float32, device="cuda")
    u = torch.empty_like(g)
    h = torch.empty((1, R), dtype=torch.int16, device="cuda")
    y = torch.full((1, C), float("nan"), dtype=torch.float32, device="cuda")
    dg.lw_gemv(dbs[0], xt, g, 1)
    dg.lw_gemv(dbs[1], xt, u, 1)
    dg.lw_swiglu(g, u, h)
    dg.lw_gemv(dbs[2], h, y, 1)
    torch.cuda.synchronize()
    gref, uref, href_bits, yref = mlp_pass_all(mats[0][:3], mats[1][:3], mats[2][:3], x, 1)
    gg, ug = g.cpu().numpy().astype(np.float64), u.cpu().numpy().astype(np.float64)
    assert rel_err(gg, gref) <= TOL and rel_err(ug, uref) <= TOL
    hr = O.swiglu(gg, ug).view(np.float16).astype(np.float64)
    hbits = h.cpu().numpy().view(np.uint16)
    hg = hbits.view(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(hr).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(hg - hr) <= ulp + 1e-12)
    yv = y.cpu().numpy()
    assert rel_err(yv, gemv_q_all(*mats[2][:3], hbits, 1)) <= TOL
    from support import activation_spread, pass_within
    assert pass_within(yv, yref, activation_spread(mats[2][:3], hbits, href_bits), TOL)


# ------------------------------------------------------------------ bf16 exponent coding

def _decode_bf16(dg, torch, db, rows, cols, n_tiles):
    out = torch.zeros(rows * cols, dtype=torch.int16, device="cuda")
    lb = torch.zeros(n_tiles * 32, dtype=torch.int32, device="cuda")
    dg.lw_decode_only(db, out, lane_bits=lb)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16).reshape(rows, cols), lb.cpu().numpy().view(np.uint32)


SMALL_BF16 = [(64, 256, 0.0, 201), (192, 768, 0.001, 202), (128, 1280, 0.02, 203), (320, 2304, 0.002, 204),
              (64, 4096, 0.0, 205)]


@pytest.mark.parametrize("case", SMALL_BF16, ids=lambda c: "-".join(map(str, c)))
def test_bf16_decode_bit_exact_small(torch, dg, case):
    rows, cols, frac, seed = case
    say("bf16 decode", case)
    w, x = synth.gen_bf16_custom(rows, cols, seed, outlier_frac=frac)
    b = dg.lw_bundle_build_bf16(w)
    info = dg.lw_bundle_get_info(b)
    if frac > 0:
        assert info["n_verbatim"] > 0
    db = _upload(dg, torch, b)
    w2, bits = _decode_bf16(dg, torch, db, rows, cols, info["n_tiles"])
    assert np.array_equal(w2, w)
    _, obits = O.decode_bundle_bf16(O.build_bundle_bf16(w))
    assert np.array_equal(bits, obits)


@pytest.mark.parametrize("case", SMALL_BF16, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("batch", [1, 3, 7])
def test_bf16_gemv_small(torch, dg, case, batch):
    rows, cols, frac, seed = case
    say("bf16 gemv", case, batch)
    w, x = synth.gen_bf16_custom(rows, cols, seed, outlier_frac=frac)
    db = _upload(dg, torch, dg.lw_bundle_build_bf16(w))
    y = _run_gemv(dg, torch, db, x, batch, rows)
    assert rel_err(y, O.gemv_bf16(w, x, batch)) <= TOL


def test_full_size_bf16(torch, dg):
    mat = synth.WORKLOADS["bf16_up_14336x4096"][0]
    say("full", mat.name)
    w, x = synth.gen_bf16(mat)
    b = dg.lw_bundle_build_bf16(w)
    info = dg.lw_bundle_get_info(b)
    db = _upload(dg, torch, b)
    w2, _ = _decode_bf16(dg, torch, db, mat.rows, mat.cols, info["n_tiles"])
    assert np.array_equal(w2, w)
    del w2
    for batch in (1, 16):
        say("full gemv", mat.name, batch)
        y = _run_gemv(dg, torch, db, x, batch, mat.rows)
        assert rel_err(y, gemv_bf16_all(w, x, batch)) <= TOL


# ------------------------------------------------------------------ batch >= 8: matrix cores

MFMA_CASES = [("q4", 64, 256, "normal", 301), ("q4", 192, 1280, "laplace", 302), ("q4", 320, 2304, "normal", 303),
              ("q6", 128, 768, "normal", 304), ("q6", 64, 2048, "uniform", 305)]


@pytest.mark.parametrize("case", MFMA_CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("batch", [8, 11, 16])
def test_gemv_mfma_small(torch, dg, case, batch):
    kind_s, rows, cols, law, seed = case
    say("mfma", case, batch)
    kind = dg.LW_Q4_PAIR if kind_s == "q4" else dg.LW_Q6_SINGLE
    codes, d, m, x = _gen_small(*case)
    db = _upload(dg, torch, dg.lw_bundle_build_q(kind, codes, d, m))
    y = _run_gemv(dg, torch, db, x, batch, rows)
    assert rel_err(y, O.gemv_q(codes, d, m, x, batch)) <= TOL
    assert np.array_equal(y, _run_gemv(dg, torch, db, x, batch, rows))



# whole-row layouts of the matrix-core kernel (sixteen wavefronts a workgroup:
# 128 row bands of 13 to 16 column blocks, bundles in one part)
MFMA_WHOLE = [("q4", 8192, 3328, "normal", 311), ("q6", 8192, 4096, "laplace", 312)]


@pytest.mark.parametrize("case", MFMA_WHOLE, ids=lambda c: "-".join(map(str, c)))
def test_gemv_mfma_whole_rows(torch, dg, case):
    kind_s, rows, cols, law, seed = case
    kind = dg.LW_Q4_PAIR if kind_s == "q4" else dg.LW_Q6_SINGLE
    codes, d, m, x = _gen_small(*case)
    db = _upload(dg, torch, dg.lw_bundle_build_q_opts(kind, codes, d, m, parts=1))
    for batch in (8, 16):
        say("mfma whole rows", case, batch)
        y = _run_gemv(dg, torch, db, x, batch, rows)
        assert rel_err(y, gemv_q_all(codes, d, m, x, batch)) <= TOL
        assert np.array_equal(y, _run_gemv(dg, torch, db, x, batch, rows))


# balanced layout: 3584 tiles (14 per CU on 256 CUs), bundles in two parts --
# whole tiles on twelve wavefronts of a CU and tile halves on four, each row
# band meeting the other workgroups holding its tiles; batch 1..4 on the
# VALU kernel, and 8 and 16 on the matrix cores' whole-row layouts over the
# same two-part bundles
BALANCED = [("q4", 14336, 4096, "normal", 321), ("q4", 4096, 14336, "laplace", 322), ("q6", 4096, 14336, "normal", 323)]


@pytest.mark.parametrize("case", BALANCED, ids=lambda c: "-".join(map(str, c)))
def test_gemv_balanced_layout(torch, dg, case):
    kind_s, rows, cols, law, seed = case
    kind = dg.LW_Q4_PAIR if kind_s == "q4" else dg.LW_Q6_SINGLE
    codes, d, m, x = _gen_small(*case)
    db = _upload(dg, torch, dg.lw_bundle_build_q_opts(kind, codes, d, m, parts=2))
    for batch in ((1, 2, 4, 8, 16) if kind_s == "q4" else (1, 16)):
        say("balanced", case, batch)
        y = _run_gemv(dg, torch, db, x, batch, rows)
        assert rel_err(y, gemv_q_all(codes, d, m, x, batch)) <= TOL
        assert np.array_equal(y, _run_gemv(dg, torch, db, x, batch, rows))

# ------------------------------------------------------------------ parts per tile row

PARTS_Q = [
    # column blocks: five (four-wavefront groups), fourteen (fourteen-wavefront
    # groups), sixteen (whole rows), eight and thirteen
    ("q4", 192, 1280, "normal", 131), ("q4", 128, 3584, "laplace", 132), ("q4", 64, 4096, "normal", 133),
    ("q6", 128, 2048, "normal", 134), ("q6", 64, 3328, "normal", 135),
]


@pytest.mark.parametrize("parts", [1, 2, 4, 8])
@pytest.mark.parametrize("case", PARTS_Q, ids=lambda c: "-".join(map(str, c)))
def test_parts_q(torch, dg, case, parts):
    """Bundles with 1, 2, 4 and 8 recorded parts per tile row: decode-only
    bit-exact (and per-lane bit counts), the VALU GEMV at batch 1, 2, 4 and 7
    and the matrix-core GEMV at batch 16 within tolerance and repeatable."""
    kind_s, rows, cols, law, seed = case
    say("parts", case, parts)
    kind = dg.LW_Q4_PAIR if kind_s == "q4" else dg.LW_Q6_SINGLE
    codes, d, m, x = _gen_small(*case)
    b = dg.lw_bundle_build_q_opts(kind, codes, d, m, parts=parts)
    info = dg.lw_bundle_get_info(b)
    assert info["parts"] == parts
    db = _upload(dg, torch, b)
    q, bits = _decode_q(dg, torch, db, kind, rows, cols, info["n_tiles"])
    assert np.array_equal(q, codes)
    _, obits = O.decode_bundle_q(O.build_bundle_q(kind, codes, d, m, parts=parts))
    assert np.array_equal(bits, obits)
    for batch in (1, 2, 4, 7, 16):
        y = _run_gemv(dg, torch, db, x, batch, rows)
        assert rel_err(y, O.gemv_q(codes, d, m, x, batch)) <= TOL, batch
        assert np.array_equal(y, _run_gemv(dg, torch, db, x, batch, rows)), batch


@pytest.mark.parametrize("parts", [1, 2, 8])
@pytest.mark.parametrize("case", [(128, 1280, 0.02, 211), (64, 4096, 0.0, 212)], ids=lambda c: "-".join(map(str, c)))
def test_parts_bf16(torch, dg, case, parts):
    rows, cols, frac, seed = case
    say("bf16 parts", case, parts)
    w, x = synth.gen_bf16_custom(rows, cols, seed, outlier_frac=frac)
    b = dg.lw_bundle_build_bf16_opts(w, parts=parts)
    info = dg.lw_bundle_get_info(b)
    assert info["parts"] == parts
    db = _upload(dg, torch, b)
    w2, _ = _decode_bf16(dg, torch, db, rows, cols, info["n_tiles"])
    assert np.array_equal(w2, w)
    for batch in (1, 3, 16):
        y = _run_gemv(dg, torch, db, x, batch, rows)
        assert rel_err(y, O.gemv_bf16(w, x, batch)) <= TOL, batch


PLAN_NAMES = {0: "compact", 1: "r2", 2: "r2k", 3: "r2x2", 4: "gen", 5: "s2k"}


def _table_for_plan(dg, want, pairs, rng):
    """A random complete code whose bundle takes comparison plan `want`."""
    kind = dg.LW_Q4_PAIR if pairs else dg.LW_Q6_SINGLE
    n_alpha = 256 if pairs else 64
    for _ in range(2000):
        n_sym = int(rng.integers(2, n_alpha + 1))
        depth = int(rng.integers(max(1, int(np.ceil(np.log2(n_sym)))), 12))
        lens, syms = random_complete_lengths(rng, n_alpha, n_sym, depth)
        probe = codes_over(rng, pairs, syms)
        z = np.zeros((64, 1), np.uint16)
        if plan_of(dg.lw_bundle_build_q_lens(kind, probe, z, z, lens))["plan"] == want:
            return lens, syms
    raise AssertionError(f"no random table takes plan {PLAN_NAMES[want]}")


@pytest.mark.parametrize("pairs", [True, False], ids=["q4", "q6"])
@pytest.mark.parametrize("plan", [0, 1, 2, 3, 4, 5], ids=lambda p: PLAN_NAMES[p])
def test_each_comparison_plan(torch, dg, plan, pairs):
    """Every comparison plan of the lane decoder on the GPU: a random complete
    code that takes it, over a matrix of several tiles with a ragged column
    group.  Decode-only restores every code with per-lane bit counts equal to
    the oracle's (its bundle built with the same lengths), and the fused GEMV
    matches the oracle at batch 1 and 3 (VALU) and 16 (matrix cores)."""
    rng = np.random.default_rng(700 + 10 * plan + pairs)
    lens, syms = _table_for_plan(dg, plan, pairs, rng)
    kind = dg.LW_Q4_PAIR if pairs else dg.LW_Q6_SINGLE
    rows, cols = (192, 1280) if pairs else (128, 768)
    say("plan", PLAN_NAMES[plan], "q4" if pairs else "q6", rows, cols)
    codes = codes_over(rng, pairs, syms, rows, cols)
    _, d, m, x = synth.gen_q_custom(rows, cols, 800 + plan)
    b = dg.lw_bundle_build_q_lens(kind, codes, d, m, lens)
    assert plan_of(b)["plan"] == plan
    info = dg.lw_bundle_get_info(b)
    db = _upload(dg, torch, b)
    q, bits = _decode_q(dg, torch, db, kind, rows, cols, info["n_tiles"])
    assert np.array_equal(q, codes)
    ok = O.Q4 if pairs else O.Q6
    _, obits = O.decode_bundle_q(O.build_bundle_q(ok, codes, d, m, lens=lens))
    assert np.array_equal(bits, obits)
    for batch in (1, 3, 16):
        y = _run_gemv(dg, torch, db, x, batch, rows)
        assert rel_err(y, O.gemv_q(codes, d, m, x, batch)) <= TOL


COMPACT_CASES = [("q4", 192, 768, "normal", 601), ("q4", 64, 4096, "normal", 602), ("q4", 128, 7168, "normal", 603),
                 ("q6", 192, 1280, "normal", 604), ("q6", 128, 3328, "normal", 605)]


@pytest.mark.parametrize("case", COMPACT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_compact_code_bundles(torch, dg, case):
    """The opt-in compact code: decode-only bit-exact with the oracle's lane
    bit counts (its compact bundle), GEMV at batch 1, 4 and 16 within 1e-3."""
    kind_s, rows, cols, law, seed = case
    say("compact", case)
    kind = dg.LW_Q4_PAIR if kind_s == "q4" else dg.LW_Q6_SINGLE
    codes, d, m, x = _gen_small(*case)
    b = dg.lw_bundle_build_q_compact(kind, codes, d, m)
    assert plan_of(b)["plan"] == 0
    info = dg.lw_bundle_get_info(b)
    db = _upload(dg, torch, b)
    q, bits = _decode_q(dg, torch, db, kind, rows, cols, info["n_tiles"])
    assert np.array_equal(q, codes)
    _, obits = O.decode_bundle_q(O.build_bundle_q(O.Q4 if kind_s == "q4" else O.Q6, codes, d, m, code="compact"))
    assert np.array_equal(bits, obits)
    for batch in (1, 4, 16):
        y = _run_gemv(dg, torch, db, x, batch, rows)
        assert rel_err(y, O.gemv_q(codes, d, m, x, batch)) <= TOL


@pytest.mark.parametrize("case", SMALL_BF16[:4], ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("batch", [8, 16])
def test_bf16_gemv_mfma_small(torch, dg, case, batch):
    rows, cols, frac, seed = case
    say("bf16 mfma", case, batch)
    w, x = synth.gen_bf16_custom(rows, cols, seed, outlier_frac=frac)
    db = _upload(dg, torch, dg.lw_bundle_build_bf16(w))
    y = _run_gemv(dg, torch, db, x, batch, rows)
    assert rel_err(y, O.gemv_bf16(w, x, batch)) <= TOL


def test_read_probe_reads_and_writes_nothing(torch, dg):
    """The measurement probe leaves its sink untouched for data whose words
    do not fold to its marker, and rejects a size that is not a multiple of 16."""
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    dg.lw_read_probe(src, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    with pytest.raises(dg.LwError):
        dg.lw_read_probe(torch.zeros(10, dtype=torch.uint8, device="cuda"), sink)
