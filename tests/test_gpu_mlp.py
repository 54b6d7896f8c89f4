"""GPU: a SwiGLU MLP pass over coded matrices through the C ABI -- lw_gemv on
the gate and up bundles, lw_swiglu, lw_gemv on the down bundle -- against the
oracle's fp64 pass.

Tolerances.  The GEMV outputs g and u, and y against the oracle's down GEMV
of the GPU's own activations h, meet the usual bar (max relative error 1e-3
with the 0.01 * rms floor).  The fp16 activations h are an fp16 rounding of
silu(g) u, computed in fp32 on the GPU and in fp64 by the oracle: on the same
g and u they can differ only where the exact value lies within the fp32
evaluation's error of a rounding boundary, i.e. by at most one fp16 ulp.
(Against the oracle's own fp64 g and u a gate output near zero carries the
fp32 sum's absolute error as a large relative error into silu.)  So y against
the oracle's whole fp64 pass differs by the GEMV error plus the down GEMV of
those activation differences: the bar there is 1e-3 plus
sum_j |w_ij| |h_j - h_ref_j|, computed from the two h vectors.
"""
import numpy as np
import pytest

import oracle as O
import synth
from support import activation_spread, mlp_pass_all, pass_within

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


def rel_err(y, ref):
    ref = np.asarray(ref, np.float64)
    floor = 0.01 * np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref) / np.maximum(np.abs(ref), floor)))


def _pass_setup(torch, dg, kind, R, C, batch, seed):
    qmax, mu, sc = (15, 7.5, 1.8) if kind == "q4" else (63, 31.5, 5.0)
    k = dg.LW_Q4_PAIR if kind == "q4" else dg.LW_Q6_SINGLE
    mats = [synth.gen_q_custom(r, c, seed + i, qmax=qmax, mu=mu, scale=sc)
            for i, (r, c) in enumerate(((R, C), (R, C), (C, R)))]
    dbs = [dg.upload(dg.lw_bundle_build_q(k, *mm[:3])) for mm in mats]
    x = mats[0][3]
    xt = torch.from_numpy(np.ascontiguousarray(x[:batch]).view(np.int16)).cuda()
    g = torch.empty((batch, R), dtype=torch.float32, device="cuda")
    u = torch.empty_like(g)
    h = torch.empty((batch, R), dtype=torch.int16, device="cuda")
    y = torch.empty((batch, C), dtype=torch.float32, device="cuda")

    def run():
        dg.lw_gemv(dbs[0], xt, g, batch)
        dg.lw_gemv(dbs[1], xt, u, batch)
        dg.lw_swiglu(g, u, h)
        dg.lw_gemv(dbs[2], h, y, batch)

    return mats, x, (g, u, h, y), run


@pytest.mark.parametrize("kind,R,C,batch", [("q4", 512, 256, 1), ("q4", 1024, 768, 3), ("q6", 512, 512, 1),
                                            ("q6", 768, 256, 3)])
def test_mlp_pass(torch, dg, kind, R, C, batch):
    print("mlp pass", kind, R, C, batch, flush=True)
    mats, x, (g, u, h, y), run = _pass_setup(torch, dg, kind, R, C, batch, 900 + R + batch)
    run()
    torch.cuda.synchronize()
    gref, uref, href_bits, ref = mlp_pass_all(mats[0][:3], mats[1][:3], mats[2][:3], x, batch)
    assert np.array_equal(ref, O.mlp_pass_q(mats[0][:3], mats[1][:3], mats[2][:3], x, batch))
    gg, ug = g.cpu().numpy().astype(np.float64), u.cpu().numpy().astype(np.float64)
    assert rel_err(gg, O.gemv_q(*mats[0][:3], x, batch)) <= 1e-3
    assert rel_err(ug, O.gemv_q(*mats[1][:3], x, batch)) <= 1e-3
    # activations: within one fp16 ulp of the oracle's SwiGLU of the same g, u
    href = O.swiglu(gg, ug).view(np.float16).astype(np.float64)
    hbits = h.cpu().numpy().view(np.uint16)
    hg = hbits.view(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(href).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(hg - href) <= ulp + 1e-12)
    assert rel_err(y.cpu().numpy(), O.gemv_q(*mats[2][:3], hbits, batch)) <= 1e-3
    # the whole pass: 1e-3 plus what the activation differences carry through down
    spread = activation_spread(mats[2][:3], hbits, href_bits)
    assert pass_within(y.cpu().numpy(), ref, spread, 1e-3)


def test_swiglu_lengths_and_alignment(torch, dg):
    # vector and scalar paths, odd lengths and offsets, n = 0
    rng = np.random.default_rng(9)
    for n, off in ((4096, 0), (4099, 0), (1, 0), (1000, 1), (0, 0)):
        print("swiglu", n, off, flush=True)
        gv = (rng.standard_normal(n + off) * 3).astype(np.float32)
        uv = (rng.standard_normal(n + off) * 3).astype(np.float32)
        g = torch.from_numpy(gv).cuda()[off:]
        u = torch.from_numpy(uv).cuda()[off:]
        h = torch.zeros(n + off, dtype=torch.int16, device="cuda")[off:]
        dg.lw_swiglu(g, u, h)
        torch.cuda.synchronize()
        ref = O.swiglu(gv[off:].astype(np.float64), uv[off:].astype(np.float64)).view(np.float16).astype(np.float64)
        got = h.cpu().numpy().view(np.float16).astype(np.float64)
        ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= ulp + 1e-12)


def test_mlp_pass_graph_replays(torch, dg):
    # the whole pass captured once and replayed: every replay equals eager
    print("mlp pass graph", flush=True)
    _, _, (g, u, h, y), run = _pass_setup(torch, dg, "q6", 512, 512, 2, 950)
    run()
    torch.cuda.synchronize()
    eager = y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for r in range(4):
        y.fill_(float("nan"))
        h.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.uint8), eager.view(torch.uint8)), f"replay {r}"
        run()                              # eager work between replays
        torch.cuda.synchronize()
