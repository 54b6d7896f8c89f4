"""CPU pins of the oracle's rANS lane coder (the decode-cost ablation of
"LazyWeights", section "Decoder hardware": Huffman against rANS).

The coder is pinned to things other than itself: hand-worked states, chunks
and frequencies (tests/golden/rans_small.txt), the information bound that the
rANS recurrence obeys exactly, round trips on every tile of synthetic
matrices of both code widths, the block layout checked stream by stream, and
degenerate alphabets."""
import math
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rans_small.txt")


def _golden(kind):
    out = []
    for line in open(GOLDEN):
        if line.startswith(kind + " "):
            out.append(dict(kv.split("=") for kv in line.split()[1:]))
    return out


def _ints(s):
    return [int(v) for v in s.split(",")] if s else []


@pytest.mark.parametrize("case", _golden("case"), ids=lambda c: c["syms"])
def test_golden_streams(case):
    f, cum, syms = (np.array(_ints(case[k]), np.uint16) for k in ("f", "cum", "syms"))
    st, ch = O.rans_encode_stream(syms, f, cum)
    want = _ints(case["state"])[0]
    assert st == want
    assert ch.tolist() == _ints(case["chunks"])
    assert O.rans_decode_stream(st, ch, syms.size, f, cum).tolist() == syms.tolist()


@pytest.mark.parametrize("case", _golden("freqs"), ids=lambda c: c["counts"])
def test_golden_freqs(case):
    f, cum = O.rans_freqs(np.array(_ints(case["counts"]), np.uint64))
    assert f.tolist() == _ints(case["f"])
    assert cum.tolist() == np.concatenate([[0], np.cumsum(f)[:-1]]).tolist()


def test_freqs_invariants():
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(1, 257))
        counts = rng.integers(0, 10 ** int(rng.integers(1, 8)), size=n).astype(np.uint64)
        if counts.sum() == 0:
            counts[int(rng.integers(n))] = 1
        f, cum = O.rans_freqs(counts)
        assert int(f.sum()) == O.RANS_M
        assert np.array_equal(f > 0, counts > 0)
        # each f is within 1 of its rounded share plus what the fix-up moved:
        # the fix-up moves at most one unit per used symbol in total
        ideal = counts.astype(np.float64) * O.RANS_M / counts.sum()
        moved = np.abs(f.astype(np.float64) - np.maximum(1, np.floor(ideal + 0.5)) * (counts > 0))
        assert moved.sum() <= (counts > 0).sum() + 1e-9


def _information(st, nchunks):
    return math.log2(st) + 16 * nchunks - 16


def test_information_bound():
    """Each coding step multiplies the state by M / f[s] up to a factor in
    (31/32, 33/32), since the state before a step is at least 32 f[s]; each
    renormalisation drops less than log2(1 + 1/32) bits.  So the information
    carried, log2(final state) + 16 * chunks - log2(L), lies within
    n log2(33/32) above and n log2(32/31) + chunks * log2(33/32) below the
    ideal sum of log2(M / f[s])."""
    rng = np.random.default_rng(11)
    for trial in range(60):
        n_alpha = int(rng.choice([2, 16, 64, 256]))
        p = rng.dirichlet(np.full(n_alpha, 0.3))
        counts = np.maximum(np.rint(p * 1e6), 0).astype(np.uint64)
        counts[0] += 1
        f, cum = O.rans_freqs(counts)
        live = np.nonzero(f)[0]
        n = int(rng.integers(1, 600))
        syms = rng.choice(live, size=n, p=f[live] / f[live].sum()).astype(np.uint16)
        st, ch = O.rans_encode_stream(syms, f, cum)
        ideal = float(np.sum(np.log2(O.RANS_M / f[syms].astype(np.float64))))
        info = _information(st, ch.size)
        assert info <= ideal + n * math.log2(33 / 32) + 1e-9
        assert info >= ideal - n * math.log2(32 / 31) - ch.size * math.log2(33 / 32) - 1e-9
        assert O.RANS_L <= st < 2 ** 32
        assert O.rans_decode_stream(st, ch, n, f, cum).tolist() == syms.tolist()


def test_single_symbol_alphabet():
    """One used symbol has f = M: coding it leaves the state at L, so a
    stream is its head state L and no chunks."""
    f, cum = O.rans_freqs(np.array([0, 0, 5, 0], np.uint64))
    assert f.tolist() == [0, 0, 2048, 0]
    st, ch = O.rans_encode_stream(np.full(300, 2, np.uint16), f, cum)
    assert st == O.RANS_L and ch.size == 0


def test_corrupt_stream_is_rejected():
    f, cum = O.rans_freqs(np.array([5, 3, 1, 1], np.uint64))
    syms = np.array([0, 1, 2, 3, 0, 0, 1, 3, 2, 1] * 20, np.uint16)
    st, ch = O.rans_encode_stream(syms, f, cum)
    with pytest.raises(ValueError):
        O.rans_decode_stream(st + 1, ch, syms.size, f, cum)
    with pytest.raises(ValueError):
        O.rans_decode_stream(st, ch[:-1], syms.size, f, cum)


@pytest.mark.parametrize("kind,law,halves", [(O.Q4, "normal", 1), (O.Q4, "uniform", 1), (O.Q4, "const", 1),
                                             (O.Q6, "normal", 1), (O.Q4, "normal", 2), (O.Q6, "uniform", 2)])
def test_tiles_round_trip_and_layout(kind, law, halves):
    rows, cols = 192, 768
    qmax, mu, sc = (15, 7.5, 1.8) if kind == O.Q4 else (63, 31.5, 5.0)
    codes, _, _, _ = synth.gen_q_custom(rows, cols, 70 + kind, qmax=qmax, law=law, mu=mu, scale=sc)
    b = O.build_rans_q(kind, codes, halves)
    assert np.array_equal(O.rans_unsymbolise(kind, rows, cols, O.decode_rans(b), halves), codes)
    ns, sps = b["ns"], b["sps"]
    assert ns == 64 * halves and sps * halves == (128 if kind == O.Q4 else 256)
    # the symbols: pairs (low nibble = even column) or single codes, by row;
    # stream h*64 + r of a tile holds half h of row r
    s = b["syms"].reshape(rows // 64, cols // 256, halves, 64, sps)
    row = codes[64 + 5, 512:768]
    want = row[0::2] | (row[1::2] << 4) if kind == O.Q4 else row
    for h in range(halves):
        assert np.array_equal(s[1, 2, h, 5], want[h * sps:(h + 1) * sps])
    # the block of every tile, stream by stream, from the stream encoder
    words = b["words"]
    for t in range(b["tile_off"].size - 1):
        blk = words[b["tile_off"][t]:b["tile_off"][t + 1]]
        streams = [O.rans_encode_stream(b["syms"][(t * ns + r) * sps:(t * ns + r + 1) * sps], b["f"], b["cum"])
                   for r in range(ns)]
        kt = max(c.size for _, c in streams)
        kt += kt & 1
        assert blk.size == ns + ns * kt // 2
        area = blk[ns:].view(np.uint16)
        for r, (st, ch) in enumerate(streams):
            assert blk[r] == st
            col = area[r::ns]
            assert np.array_equal(col[:ch.size], ch) and not col[ch.size:].any()


def test_bits_close_to_the_huffman_code():
    """On the 4-bit workload law the rANS symbol information is at least the
    entropy (Gibbs' inequality: the excess is the divergence of f / M from
    the histogram) and, measured, within 2 % of it (2.950 against 2.913 bits
    per weight); the coded words (head states and padding included) stay
    within 10 % of the Huffman bundle's words (3.23 against 3.10 bits per
    weight), so the ablation compares decoders at almost the same rate."""
    codes, d, m, _ = synth.gen_q_custom(512, 4096, 90)
    r = O.build_rans_q(O.Q4, codes)
    h = O.build_bundle_q(O.Q4, codes, d, m)
    p = r["counts"][r["counts"] > 0].astype(np.float64)
    p /= p.sum()
    ent = float(-(p * np.log2(p)).sum()) * r["syms"].size
    ideal = float(np.sum(np.log2(O.RANS_M / r["f"][r["syms"]].astype(np.float64))))
    assert ent <= ideal <= 1.02 * ent
    assert r["words"].size <= 1.10 * h["words"].size
