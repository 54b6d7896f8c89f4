"""GPU parity of the rANS twin's decode-only kernel (lw_rans_decode), the
decode-cost ablation of "LazyWeights" (section "Decoder hardware": Huffman
against rANS decoders).

The kernel must restore the fixed-width codes exactly (byte for byte: Q4
nibble pairs, low nibble the even column, or one Q6 code per byte), and every
stream must end in the state 2^16 that the oracle's decoder requires.  The
words come from the product builder, which test_builder checks bit for bit
against the oracle's encoder; the oracle's own decoder restores the same
codes from them here too on the small cases."""
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


def say(*a):
    print(*a, flush=True)


def packed(kind_q4, codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8) if kind_q4 else codes.astype(np.uint8)


def run(dg, torch, kind, codes, r=None, max_tile_words=None, sentinel=0xA5, halves=1):
    rows, cols = codes.shape
    r = r or dg.lw_rans_build(kind, codes, halves)
    halves = r["halves"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()
    lut, to, w = dev(r["lut"]), dev(r["tile_off"]), dev(r["words"] if r["words"].size else np.zeros(4, np.uint32))
    ob = rows * cols // 2 if kind == dg.LW_Q4_PAIR else rows * cols
    out = torch.full((ob,), sentinel, dtype=torch.uint8, device="cuda")
    nt = (rows // 64) * (cols // 256)
    fs = torch.zeros(nt * 64 * halves, dtype=torch.int32, device="cuda")
    dg.lw_rans_decode(kind, rows, cols, lut, to, w, max_tile_words or r["max_tile_words"], out, fs, halves)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(rows, -1), fs.cpu().numpy().view(np.uint32), r


def qlaw(kind, dg):
    return (15, 7.5, 1.8) if kind == dg.LW_Q4_PAIR else (63, 31.5, 5.0)


CASES = [  # kind (1 = Q4, 2 = Q6), law, rows, cols, seed: one tile, ragged workgroup tails (tiles not a
           # multiple of 4), uniform codes (longest streams), one symbol (no chunks at all)
    (1, "normal", 64, 256, 1), (1, "normal", 192, 768, 2), (1, "uniform", 128, 1280, 3),
    (1, "const", 64, 512, 4), (1, "laplace", 320, 2304, 5), (2, "normal", 64, 256, 6),
    (2, "normal", 192, 1792, 7), (2, "uniform", 128, 512, 8), (2, "const", 64, 768, 9),
]


@pytest.mark.parametrize("halves", [1, 2])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"k{c[0]}_{c[1]}_{c[2]}x{c[3]}")
def test_rans_decode_restores_codes(torch, dg, case, halves):
    kind, law, rows, cols, seed = case
    say("rans decode", case, halves)
    qmax, mu, sc = qlaw(kind, dg)
    codes, _, _, _ = synth.gen_q_custom(rows, cols, seed, qmax=qmax, law=law, mu=mu,
                                        scale=1.2 if law == "laplace" else sc)
    out, fs, r = run(dg, torch, kind, codes, halves=halves)
    assert np.array_equal(out, packed(kind == dg.LW_Q4_PAIR, codes))
    assert np.all(fs == 65536)
    ob = O.build_rans_q(O.Q4 if kind == dg.LW_Q4_PAIR else O.Q6, codes, halves)
    assert np.array_equal(O.rans_unsymbolise(ob["kind"], rows, cols, O.decode_rans(ob), halves), codes)


def test_rans_decode_twice_is_identical(torch, dg):
    codes, _, _, _ = synth.gen_q_custom(256, 1024, 21)
    a, _, r = run(dg, torch, dg.LW_Q4_PAIR, codes)
    b, _, _ = run(dg, torch, dg.LW_Q4_PAIR, codes, r=r, sentinel=0x11)
    assert np.array_equal(a, b)


def test_rans_blocks_beyond_the_limit_are_skipped(torch, dg):
    """A max_tile_words below some blocks: those tiles are left untouched (the
    sentinel), the others decode exactly."""
    rows, cols = 128, 1024
    codes, _, _, _ = synth.gen_q_custom(rows, cols, 22, law="uniform")
    codes[:64, :256] = 7                                  # tile 0: one symbol, the smallest block
    r = dg.lw_rans_build(dg.LW_Q4_PAIR, codes)
    sizes = np.diff(r["tile_off"].astype(np.int64))
    lim = int(sizes.min())
    assert lim < sizes.max()
    out, _, _ = run(dg, torch, dg.LW_Q4_PAIR, codes, r=r, max_tile_words=lim)
    want = packed(True, codes)
    ncb = cols // 256
    for t, n in enumerate(sizes):
        blk = (slice(64 * (t // ncb), 64 * (t // ncb) + 64), slice(128 * (t % ncb), 128 * (t % ncb) + 128))
        if n <= lim:
            assert np.array_equal(out[blk], want[blk])
        else:
            assert np.all(out[blk] == 0xA5)


@pytest.mark.parametrize("halves", [1, 2])
def test_rans_corrupt_words_stay_in_bounds(torch, dg, halves):
    """Random words under valid offsets decode to garbage codes and final
    states other than 2^16, touching only the output."""
    codes, _, _, _ = synth.gen_q_custom(128, 512, 23)
    r = dg.lw_rans_build(dg.LW_Q4_PAIR, codes, halves)
    r = dict(r)
    r["words"] = np.random.default_rng(24).integers(0, 2 ** 32, size=r["words"].size, dtype=np.uint64).astype(np.uint32)
    out, fs, _ = run(dg, torch, dg.LW_Q4_PAIR, codes, r=r)
    assert out.shape == (128, 256)
    assert np.mean(fs != 65536) > 0.9


@pytest.mark.parametrize("halves", [1, 2])
@pytest.mark.parametrize("name", ["q4_up_14336x4096", "q6_gate_28672x8192"])
def test_rans_full_size(torch, dg, name, halves):
    """The 14336x4096 4-bit matrix and one 28672x8192 6-bit 70B matrix: every
    code restored and every stream ending in 2^16."""
    mat = next(m for ms in synth.WORKLOADS.values() for m in ms if m.name == name)
    say("rans full", name, halves)
    codes, _, _, _ = synth.gen_q(mat)
    kind = dg.LW_Q4_PAIR if mat.kind == "q4" else dg.LW_Q6_SINGLE
    out, fs, _ = run(dg, torch, kind, codes, halves=halves)
    assert np.array_equal(out, packed(kind == dg.LW_Q4_PAIR, codes))
    assert np.all(fs == 65536)
