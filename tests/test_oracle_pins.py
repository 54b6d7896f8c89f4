"""Pins of the CPU oracle against facts fixed by the pages or by mathematics.

None of these tests restates the oracle's own code: each checks it against an
independent definition (Kraft's equality, exhaustive search for optimal
lengths, the dyadic closed form, a textbook heap Huffman, brute-force bit
strings, numpy's fp16 conversion, a dense numpy matvec, closed-form special
cases, a hand-worked example) so that a dropped term, a wrong index or a
transposed operand anywhere in the oracle fails one of them.
"""
import heapq
import itertools
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def kraft_sum(lens, L=11):
    return int(sum(1 << (L - int(x)) for x in lens if x))


def heap_huffman_cost(counts):
    """Textbook Huffman (repeatedly merge the two lightest): total cost."""
    h = [int(c) for c in counts if c > 0]
    if len(h) == 1:
        return h[0]
    heapq.heapify(h)
    cost = 0
    while len(h) > 1:
        a = heapq.heappop(h)
        b = heapq.heappop(h)
        cost += a + b
        heapq.heappush(h, a + b)
    return cost


def heap_huffman_maxlen(counts):
    h = [(int(c), 0, i) for i, c in enumerate(counts) if c > 0]
    heapq.heapify(h)
    uid = len(counts)
    depth = {}
    while len(h) > 1:
        a = heapq.heappop(h)
        b = heapq.heappop(h)
        d = max(a[1], b[1]) + 1
        heapq.heappush(h, (a[0] + b[0], d, uid))
        uid += 1
    return h[0][1]


def brute_force_opt(counts, L):
    """Minimum sum(count*len) over all length vectors with Kraft <= 1, max <= L.

    With counts sorted descending an optimal vector is non-decreasing (swapping
    two lengths onto the heavier symbol never costs more), so the search runs
    over non-decreasing vectors only, which still contains an optimum."""
    used = sorted((int(c) for c in counts if c > 0), reverse=True)
    best = None
    for lens in itertools.combinations_with_replacement(range(1, L + 1), len(used)):
        if sum(1 << (L - l) for l in lens) <= (1 << L):
            cost = sum(c * l for c, l in zip(used, lens))
            best = cost if best is None else min(best, cost)
    return best


# ------------------------------------------------------------------ lengths

def test_golden_hand_worked_table():
    rows = {}
    for line in open(os.path.join(GOLDEN, "canonical_small.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            rows[k] = [int(t) for t in v]
    lens = O.package_merge(np.array(rows["counts"], np.uint64))
    assert lens.tolist() == rows["lens"]
    tab = O.canonical(lens)
    assert tab["codes"].tolist() == rows["codes"]
    for k in ("count", "first", "limit", "offset"):
        assert tab[k].tolist() == rows[k], k
    assert tab["sym_sorted"].tolist() == rows["sym_sorted"]
    assert O.package_merge(np.array(rows["tie_counts"], np.uint64)).tolist() == rows["tie_lens"]


@pytest.mark.parametrize("seed", range(40))
def test_package_merge_is_optimal_small(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 8))
    counts = rng.integers(1, 60, size=n).astype(np.uint64)
    if seed % 3 == 0:
        counts = np.array(sorted(counts)[::-1], np.uint64) ** 2  # skewed
    for L in (3, 4, 11):
        if (1 << L) < n:
            continue
        lens = O.package_merge(counts, L)
        assert max(lens) <= L
        assert sum(2.0 ** -int(l) for l in lens) <= 1.0
        assert int(np.dot(counts, lens.astype(np.uint64))) == brute_force_opt(counts.tolist(), L)


def test_dyadic_closed_form():
    # counts proportional to 2^-k give lengths exactly k (the last two share k)
    for kmax in range(2, 12):
        counts = [1 << (kmax - k) for k in range(1, kmax)] + [1]
        lens = O.package_merge(np.array(counts, np.uint64))
        expect = list(range(1, kmax)) + [kmax - 1]
        assert lens.tolist() == expect


@pytest.mark.parametrize("seed", range(10))
def test_equals_heap_huffman_when_limit_slack(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 129))
    counts = rng.integers(20000, 100000, size=n).astype(np.uint64)
    assert heap_huffman_maxlen(counts) <= 11
    lens = O.package_merge(counts)
    assert int(np.dot(counts, lens.astype(np.uint64))) == heap_huffman_cost(counts)
    assert kraft_sum(lens) == 2048


def test_fibonacci_limit_binds():
    fib = [1, 1]
    while len(fib) < 25:
        fib.append(fib[-1] + fib[-2])
    counts = np.array(fib, np.uint64)
    assert heap_huffman_maxlen(counts) > 11
    lens = O.package_merge(counts)
    assert max(lens) == 11
    assert kraft_sum(lens) == 2048
    # optimality against a small limit by brute force on a prefix of the chain
    small = np.array(fib[:7], np.uint64)
    assert int(np.dot(small, O.package_merge(small, 4).astype(np.uint64))) == \
        brute_force_opt(small.tolist(), 4)


def test_degenerate_alphabets():
    one = np.zeros(256, np.uint64); one[37] = 999
    lens = O.package_merge(one)
    assert lens[37] == 1 and lens.sum() == 1
    two = np.zeros(256, np.uint64); two[[3, 200]] = [5, 7]
    assert sorted(O.package_merge(two)[[3, 200]].tolist()) == [1, 1]
    uni = np.full(256, 10, np.uint64)
    assert (O.package_merge(uni) == 8).all()
    with pytest.raises(ValueError):
        O.package_merge(np.ones(300, np.uint64), 8)     # 300 symbols cannot fit 8 bits


# ------------------------------------------------------------------ canonical

def _bitstr(code, n):
    return format(int(code), "0%db" % n) if n else ""


@pytest.mark.parametrize("seed", range(8))
def test_canonical_prefix_free_and_ordered(seed):
    rng = np.random.default_rng(200 + seed)
    counts = rng.integers(0, 5000, size=256).astype(np.uint64) ** 2
    lens = O.package_merge(counts)
    tab = O.canonical(lens)
    words = {s: _bitstr(tab["codes"][s], lens[s]) for s in range(256) if lens[s]}
    vals = list(words.values())
    for a in vals:                       # prefix-free, brute force
        for b in vals:
            assert a == b or not b.startswith(a)
    # order: (len, sym) ascending is numeric order of left-justified codes
    order = sorted(words, key=lambda s: (lens[s], s))
    lj = [int(words[s], 2) << (11 - int(lens[s])) for s in order]
    assert lj == sorted(lj) and len(set(lj)) == len(lj)
    assert tab["sym_sorted"].tolist() == order
    # limits are non-decreasing and close at 2048 for a complete code
    lim = tab["limit"][1:].astype(int)
    assert (np.diff(lim) >= 0).all() and lim[-1] == 2048
    assert kraft_sum(lens) == 2048


@pytest.mark.parametrize("seed", range(4))
def test_canonical_equals_greedy_search(seed):
    """The canonical assignment (RFC 1951, section 3.2.2: codes of one length
    consecutive in symbol order, shorter lengths first) found by search
    instead of the recurrence: in (length, symbol) order, each symbol takes
    the smallest code of its length that no earlier code is a prefix of and
    that lies above every earlier code left-justified to 11 bits.  Random
    length vectors, complete and incomplete (Kraft sum below 1)."""
    rng = np.random.default_rng(300 + seed)
    for trial in range(60):
        n = int(rng.integers(1, 13))
        while True:
            lens = np.zeros(16, np.uint8)
            lens[rng.choice(16, n, replace=False)] = rng.integers(1, 12, n)
            if kraft_sum(lens) <= 2048:
                break
        tab = O.canonical(lens)
        taken = []
        for sym in sorted(np.flatnonzero(lens), key=lambda s: (int(lens[s]), s)):
            L = int(lens[sym])
            floor = max((int(c, 2) << (11 - len(c)) for c in taken), default=-1)
            for v in range(1 << L):
                c = format(v, f"0{L}b")
                if (int(c, 2) << (11 - L)) > floor and not any(c.startswith(t) or t.startswith(c) for t in taken):
                    break
            else:
                raise AssertionError("no code left")
            taken.append(c)
            assert _bitstr(tab["codes"][sym], L) == c, (lens.tolist(), sym)


# ------------------------------------------------------------------ streams

def _bundle_bits_by_hand(syms, spl, lens, codes, nt):
    """Each lane's stream as a bit string built from the code table."""
    out = []
    s = syms.reshape(nt, 32, spl)
    for t in range(nt):
        out.append(["".join(_bitstr(codes[v], lens[v]) for v in s[t, l]) for l in range(32)])
    return out


@pytest.mark.parametrize("kind,law,seed", [(O.Q4, "normal", 1), (O.Q4, "laplace", 2),
                                            (O.Q6, "normal", 3), (O.Q4, "uniform", 4),
                                            (O.Q4, "const", 5)])
def test_interleave_matches_bit_strings(kind, law, seed):
    qmax = 15 if kind == O.Q4 else 63
    mu = 31.5 if kind == O.Q6 else 7.5
    codes, d, m, _ = synth.gen_q_custom(128, 512, seed, qmax=qmax, law=law, mu=mu,
                                        scale=5.0 if kind == O.Q6 else 1.8)
    b = O.build_bundle_q(kind, codes, d, m)
    nt = 4
    spl = b["spl"]
    tab = b["table"]
    syms = O.symbolise_q(kind, codes)
    hand = _bundle_bits_by_hand(syms, spl, tab["lens"], tab["codes"], nt)
    toff = b["tile_off"].astype(int)
    assert toff[0] == 0 and (np.diff(toff) % 32 == 0).all() and (np.diff(toff) > 0).all()
    for t in range(nt):
        blk = b["words"][toff[t]:toff[t + 1]].reshape(-1, 32)     # [j][lane]
        W = blk.shape[0]
        nwords = [(len(hand[t][l]) + 31) // 32 for l in range(32)]
        assert W == max(nwords)                      # padded to the longest lane
        for l in range(32):
            bits = "".join(format(int(w), "032b") for w in blk[:, l])
            assert bits[:len(hand[t][l])] == hand[t][l]
            assert set(bits[len(hand[t][l]):]) <= {"0"}
            assert b["lane_bits"][t * 32 + l] == len(hand[t][l])


def test_symbol_order_by_hand():
    codes = np.arange(64 * 256, dtype=np.int64).reshape(64, 256) % 16
    codes = codes.astype(np.uint8)
    codes[5, 10] = 3
    syms = O.symbolise_q(O.Q4, codes).reshape(32, 256)
    # lane 2 holds rows 4 and 5; its symbol 128 + 5 is row 5 columns 10 (low), 11 (high)
    assert syms[2, 128 + 5] == (codes[5, 10] | (codes[5, 11] << 4))
    assert syms[7, 3] == (codes[14, 6] | (codes[14, 7] << 4))
    s6 = O.symbolise_q(O.Q6, codes).reshape(32, 512)
    assert s6[2, 256 + 10] == codes[5, 10] and s6[31, 255] == codes[62, 255]


@pytest.mark.parametrize("kind,rows,cols,law,seed", [
    (O.Q4, 64, 256, "normal", 11), (O.Q4, 192, 768, "normal", 12),
    (O.Q4, 128, 1024, "laplace", 13), (O.Q6, 128, 512, "normal", 14),
    (O.Q4, 64, 512, "uniform", 15), (O.Q4, 64, 256, "const", 16),
    (O.Q6, 64, 256, "const", 17)])
def test_round_trip_every_tile_and_bitwise(kind, rows, cols, law, seed):
    qmax = 15 if kind == O.Q4 else 63
    codes, d, m, _ = synth.gen_q_custom(rows, cols, seed, qmax=qmax, law=law,
                                        mu=31.5 if kind == O.Q6 else 7.5,
                                        scale=5.0 if kind == O.Q6 else 1.8)
    b = O.build_bundle_q(kind, codes, d, m)
    q1, bits = O.decode_bundle_q(b)
    assert np.array_equal(q1, codes)
    assert np.array_equal(bits, b["lane_bits"])
    q2, _ = O.decode_bundle_q(b, bitwise=True)
    assert np.array_equal(q2, codes)
    # consumed bits equal the sum of code lengths of the lane's symbols
    syms = O.symbolise_q(kind, codes).reshape(-1, b["spl"])
    assert np.array_equal(b["table"]["lens"][syms].astype(np.int64).sum(1), bits.astype(np.int64))


def test_round_trip_reduced_workloads():
    for wl, kind in (("q4_up_14336x4096", O.Q4), ("q4_down_4096x14336", O.Q4), ("q6_mlp_70b", O.Q6)):
        mat = synth.WORKLOADS[wl][0]
        codes, d, m, _ = synth.gen_q(mat, rows=256, cols=2048)
        b = O.build_bundle_q(kind, codes, d, m)
        q, _ = O.decode_bundle_q(b)
        assert np.array_equal(q, codes)
        assert b["table"]["lens"].max() <= 11


def test_dm_layout():
    _, d, m, _ = synth.gen_q_custom(128, 512, 21)
    dm = O.pack_dm(d, m).reshape(2, 2, 64)            # [rb][cb][row]
    assert dm[1, 0, 5] == (int(d[69, 0]) | int(m[69, 0]) << 16)
    assert dm[0, 1, 63] == (int(d[63, 1]) | int(m[63, 1]) << 16)


# ------------------------------------------------------------------ numerics

def test_half_and_bf16_conversions_exact():
    h = np.arange(65536, dtype=np.uint16)
    f = h.view(np.float16).astype(np.float64)
    ok = ~np.isnan(f)
    got = np.array([O.half_to_double(int(v)) for v in h[ok][::7]])
    assert np.array_equal(got, f[ok][::7])
    b = np.arange(0, 65536, 5, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        fb = (b << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    ok = ~np.isnan(fb)
    got = np.array([O.bf16_to_double(int(v)) for v in b[ok]])
    assert np.array_equal(got, fb[ok])


def _dense_w(codes, d, m):
    R, Cc = codes.shape
    dd = np.repeat(d.view(np.float16).astype(np.float64), 256, axis=1)
    mm = np.repeat(m.view(np.float16).astype(np.float64), 256, axis=1)
    return dd * codes.astype(np.float64) - mm


@pytest.mark.parametrize("batch", [1, 3])
def test_gemv_vs_dense_numpy(batch):
    codes, d, m, x = synth.gen_q_custom(128, 768, 31)
    y = O.gemv_q(codes, d, m, x, batch)
    ref = x[:batch].view(np.float16).astype(np.float64) @ _dense_w(codes, d, m).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    rows = np.array([0, 5, 127, 64])
    ys = O.gemv_q(codes, d, m, x, batch, rows=rows)
    np.testing.assert_array_equal(ys, y[:, rows])


def test_gemv_special_cases():
    codes, d, m, x = synth.gen_q_custom(64, 512, 32)
    W = _dense_w(codes, d, m)
    for c in (0, 255, 256, 511):
        e = np.zeros((1, 512), np.float16); e[0, c] = 1.0
        y = O.gemv_q(codes, d, m, e.view(np.uint16), 1)
        assert np.array_equal(y[0], W[:, c])            # exact column
    eight = np.full_like(codes, 8)
    assert np.array_equal(O.gemv_q(eight, d, m, x, 2), np.zeros((2, 64)))   # m = 8d
    # idempotent codec: round((w + m) / d) recovers every code exactly
    dd = np.repeat(d.view(np.float16).astype(np.float64), 256, axis=1)
    mm = np.repeat(m.view(np.float16).astype(np.float64), 256, axis=1)
    assert np.array_equal(np.rint((W + mm) / dd).astype(np.uint8), codes)


def test_gemv_bf16_vs_dense():
    w, x = synth.gen_bf16_custom(64, 512, 41)
    y = O.gemv_bf16(w, x, 2)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf = (x[:2].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(y, xf @ wf.T, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ bf16

@pytest.mark.parametrize("frac,seed", [(0.0, 51), (0.0005, 52), (0.01, 53)])
def test_bf16_bit_exact_and_verbatim(frac, seed):
    w, _ = synth.gen_bf16_custom(128, 512, seed, outlier_frac=frac)
    b = O.build_bundle_bf16(w)
    # palette: the 16 most frequent exponents, count desc then exponent asc
    e = ((w >> 7) & 0xFF).astype(np.int64).ravel()
    cnt = np.bincount(e, minlength=256)
    order = np.lexsort((np.arange(256), -cnt))
    order = [v for v in order if cnt[v] > 0][:16]
    assert b["palette"][:len(order)].tolist() == order
    # verbatim segments: exactly the 64-wide row runs with an exponent outside
    inpal = np.zeros(256, bool); inpal[order] = True
    seg_out = (~inpal[e.reshape(128, 512)]).reshape(128, 8, 64).any(-1)
    assert b["n_verbatim"] == int(seg_out.sum())
    for dec in (False, True):
        w2, _ = O.decode_bundle_bf16(b, bitwise=dec)
        assert np.array_equal(w2, w)


def test_bf16_exponent_statistics():
    # "Unweight": more than 99 % of a layer's weights use one of its 16
    # commonest exponents, whose distribution carries about 2.6 bits
    mat = synth.WORKLOADS["bf16_up_14336x4096"][0]
    w, _ = synth.gen_bf16(mat, rows=512, cols=4096)
    e = ((w >> 7) & 0xFF).ravel()
    cnt = np.bincount(e, minlength=256).astype(np.float64)
    p = np.sort(cnt)[::-1] / cnt.sum()
    assert p[:16].sum() > 0.99
    H = -(p[p > 0] * np.log2(p[p > 0])).sum()
    assert 2.3 < H < 2.9
    b = O.build_bundle_bf16(w)
    w2, _ = O.decode_bundle_bf16(b)
    assert np.array_equal(w2, w)


def test_rejects_bad_shapes():
    codes = np.zeros((65, 256), np.uint8)
    with pytest.raises(ValueError):
        O.build_bundle_q(O.Q4, codes, np.zeros((65, 1), np.uint16), np.zeros((65, 1), np.uint16))


def _lane_bits(words, tile_off, t, l):
    """Bit string of lane l of tile t (MSB-first words at tile_off[t] + 32 j + l)."""
    w0, w1 = int(tile_off[t]), int(tile_off[t + 1])
    out = []
    for j in range((w1 - w0) // 32):
        v = int(words[w0 + 32 * j + l])
        out.extend((v >> (31 - i)) & 1 for i in range(32))
    return out


def _bitwise_from(bits, start, n, code_map):
    """Decode n symbols bit by bit from position start; returns (symbols, end)."""
    pos, syms = start, []
    for _ in range(n):
        code, ln = 0, 0
        while True:
            code = (code << 1) | bits[pos]
            pos += 1
            ln += 1
            assert ln <= 11
            if (ln, code) in code_map:
                syms.append(code_map[(ln, code)])
                break
    return syms, pos


@pytest.mark.parametrize("parts", [1, 2, 4, 8])
@pytest.mark.parametrize("case", ["q4", "q6", "bf16"])
def test_part_starts_mark_runs(case, parts):
    # with 2*parts runs of spl/(2*parts) symbols per lane stream (parts per
    # tile row), the recorded start of run k is where decoding run k-1 from
    # its own start ends, and decoding from there yields exactly run k's
    # symbols (checked with a bit-at-a-time decoder); with one part per row
    # the only start is the second tile row's
    if case == "bf16":
        w, _ = synth.gen_bf16_custom(64, 512, 77, outlier_frac=0.01)
        b = O.build_bundle_bf16(w, parts=parts)
        spl = 512
        syms = O.symbolise_bf16(w, b["palette"], b["n_pal"], b["vb_bits"])
    else:
        kind = O.Q4 if case == "q4" else O.Q6
        codes, d, m, _ = synth.gen_q_custom(64, 512, 78, qmax=15 if case == "q4" else 63,
                                            mu=7.5 if case == "q4" else 31.5, scale=1.8 if case == "q4" else 5.0)
        b = O.build_bundle_q(kind, codes, d, m, parts=parts)
        spl = b["spl"]
        syms = O.symbolise_q(kind, codes)
    assert b["parts"] == parts
    syms = syms.reshape(-1, 32, spl)
    lens, cw = b["table"]["lens"], b["table"]["codes"]
    code_map = {(int(lens[s]), int(cw[s])): s for s in range(len(lens)) if lens[s] > 0}
    nrun, per = 2 * parts, spl // (2 * parts)
    starts = b["split"].reshape(syms.shape[0], nrun - 1, 32)
    if parts == 1:
        assert np.array_equal(b["split"], O.row_split(syms.ravel(), spl, lens))
    for t in range(syms.shape[0]):
        for l in (0, 5, 17, 31):
            bits = _lane_bits(b["words"], b["tile_off"], t, l)
            pos = 0
            for k in range(nrun):
                if k:
                    assert pos == starts[t, k - 1, l]
                run, pos = _bitwise_from(bits, int(starts[t, k - 1, l]) if k else 0, per, code_map)
                assert run == list(syms[t, l, k * per:(k + 1) * per])


def test_default_parts_rule():
    # the largest of 8, 4, 2 that keeps tiles x parts within 4096 units, else 1
    assert [O.default_parts(n) for n in (1, 16, 512, 513, 1024, 1025, 2048, 2049, 3584, 14336)] == \
        [8, 8, 8, 4, 4, 2, 2, 1, 1, 1]
    # 4- and 6-bit codes: 2 where the tiles are an odd multiple of 512 in
    # (2048, 4096] and a row band has more than 16 column blocks
    q = lambda n, cb: O.default_parts(n, cb, quantised=True)
    assert [q(3584, 56), q(2560, 40), q(3584, 16), q(3072, 48), q(4096, 64), q(3584, 17), q(14336, 112)] == \
        [2, 2, 1, 1, 1, 2, 1]
    assert q(1024, 16) == 4 and O.default_parts(3584, 56) == 1      # bf16 keeps the tile-count rule


def test_double_to_half_matches_numpy_rounding():
    # or_double_to_half against numpy's correctly rounded float64 -> float16
    # conversion: every fp16 value, every midpoint between neighbours (ties
    # go to even), random values over the normal, subnormal and overflow
    # ranges, signed zeros and infinities
    allh = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = allh.view(np.float16).astype(np.float64)
    vals = vals[np.isfinite(vals)]
    srt = np.unique(vals)
    mids = (srt[:-1] + srt[1:]) / 2
    rng = np.random.default_rng(5)
    rnd = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                          rng.uniform(65000, 70000, 200), -rng.uniform(65000, 70000, 200),
                          [0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25,
                           3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -26]])
    for v in np.concatenate([vals, mids, rnd]):
        want = int(np.float64(v).astype(np.float16).view(np.uint16))
        assert O.double_to_half(float(v)) == want, (v, hex(want))


def test_swiglu_matches_expit():
    # h = fp16(silu(g) u), silu(z) = z * sigmoid(z) with scipy's logistic
    from scipy.special import expit
    rng = np.random.default_rng(6)
    g = np.concatenate([rng.standard_normal(5000) * 3, [0.0, 30.0, -30.0, 1e-6, -1e-6]])
    u = np.concatenate([rng.standard_normal(5000) * 3, [2.0, 1.5, 7.0, 1.0, 1.0]])
    want = (g * expit(g) * u).astype(np.float16).view(np.uint16)
    assert np.array_equal(O.swiglu(g, u), want)
    assert O.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0           # silu(0) = 0


@pytest.mark.parametrize("kind", ["q4", "q6"])
def test_mlp_pass_vs_dense(kind):
    # the oracle's MLP pass against dense fp64 matrices materialised as d*q - m
    from scipy.special import expit
    qmax = 15 if kind == "q4" else 63
    mu, sc = (7.5, 1.8) if kind == "q4" else (31.5, 5.0)
    R, C = 512, 256                       # gate, up: R x C; down: C x R
    gate = synth.gen_q_custom(R, C, 81, qmax=qmax, mu=mu, scale=sc)
    up = synth.gen_q_custom(R, C, 82, qmax=qmax, mu=mu, scale=sc)
    down = synth.gen_q_custom(C, R, 83, qmax=qmax, mu=mu, scale=sc)
    x = gate[3]

    def dense(codes, d, m):
        df = np.repeat(d.view(np.float16).astype(np.float64), 256, axis=1)
        mf = np.repeat(m.view(np.float16).astype(np.float64), 256, axis=1)
        return df * codes - mf

    xf = x[:2].view(np.float16).astype(np.float64)
    g = xf @ dense(*gate[:3]).T
    u = xf @ dense(*up[:3]).T
    h = (g * expit(g) * u).astype(np.float16).astype(np.float64)
    want = h @ dense(*down[:3]).T
    got = O.mlp_pass_q(gate[:3], up[:3], down[:3], x, 2)
    assert np.allclose(got, want, rtol=1e-9, atol=1e-9 * np.abs(want).max())


# ------------------------------------------------- tile-skipping fixed-width twin

def _skip_golden():
    rows = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "skip_layout.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_skip_layout_golden():
    """Words and scales of the tile-transposed layout against the hand-worked
    values of tests/golden/skip_layout.txt ("Software-Defined Bandwidth
    Expansion" IV-A, IV-B)."""
    R, Cc = 128, 256
    rr, cc = np.meshgrid(np.arange(R), np.arange(Cc), indexing="ij")
    d = np.arange(R, dtype=np.uint16).reshape(R, 1)
    m = (1000 + np.arange(R)).astype(np.uint16).reshape(R, 1)
    packed = {}
    for bits in (2, 4, 8):
        packed[bits] = O.skip_pack(((rr + cc) % (1 << bits)).astype(np.uint8), bits, d, m)
    n = 0
    for f in _skip_golden():
        if f[0] == "dm":
            r, want = int(f[1]), int(f[2], 16)
            assert packed[4][1][((r // 64) * 1 + 0) * 64 + r % 64] == want
        else:
            bits, r, j, want = int(f[0]), int(f[1]), int(f[2]), int(f[3], 16)
            wpr = Cc // (32 // bits)
            got = packed[bits][0][((r // 64) * wpr + j) * 64 + r % 64]
            assert got == want, (bits, r, j, hex(int(got)), hex(want))
        n += 1
    assert n == 13


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_skip_gemv_all_tiles_is_dense(bits):
    """With every tile listed the packed GEMV is the dense dequantise-then-
    multiply product over the original codes (IV-C's validation)."""
    codes, d, m, x = synth.gen_fixed(192, 768, bits, 40 + bits)
    words, dm = O.skip_pack(codes, bits, d, m)
    y = O.skip_gemv(words, dm, bits, 192, 768, np.arange(3), x, 2)
    ref = O.gemv_q(codes, d, m, x, 2)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_skip_gemv_skips_and_touches_only_listed_tiles():
    """Rows of unlisted tiles are not written; repeated entries give the same
    rows and out-of-range entries name no tile; words outside the listed
    tiles do not enter the result, and the listed tiles hold exactly
    n_active * WPR * B_N words (the IV-C ledger)."""
    bits, R, Cc = 4, 64 * 8, 512
    codes, d, m, x = synth.gen_fixed(R, Cc, bits, 77)
    words, dm = O.skip_pack(codes, bits, d, m)
    tiles = np.array([5, 1, 6, 1, -1, 8, 1000], dtype=np.int32)      # 3 distinct valid tiles + junk
    active = [1, 5, 6]
    y = O.skip_gemv(words, dm, bits, R, Cc, tiles, x, 1)
    ref = O.gemv_q(codes, d, m, x, 1)
    for t in range(R // 64):
        sl = slice(64 * t, 64 * t + 64)
        if t in active:
            np.testing.assert_allclose(y[0, sl], ref[0, sl], rtol=1e-12, atol=1e-12)
        else:
            assert np.all(np.isnan(y[0, sl]))
    wpr = Cc // (32 // bits)
    poisoned = np.full_like(words, 0xFFFFFFFF)
    kept = 0
    for t in active:
        sl = slice(t * wpr * 64, (t + 1) * wpr * 64)
        poisoned[sl] = words[sl]
        kept += sl.stop - sl.start
    y2 = O.skip_gemv(poisoned, dm, bits, R, Cc, np.array(active, np.int32), x, 1)
    np.testing.assert_array_equal(np.nan_to_num(y2, nan=7.0), np.nan_to_num(y, nan=7.0))
    assert kept == O.skip_ledger(Cc, bits, len(active), 1)["words"] == len(active) * wpr * 64


def test_skip_ledger_page_configuration():
    """IV-C's worked configuration (1024 output rows, K = 4096, 2-bit codes,
    64-row tiles, 6 tiles of the 16 active): words touched n_active * WPR * B_N with
    WPR = K / 16 = 256, i.e. 98304 words; against a dense fp16 pass of the
    whole matrix (8 MiB) the weight words alone are 1/64 of the bytes at full
    activity (16 bits per weight -> 2) times 6/16."""
    L = O.skip_ledger(4096, 2, 6, 1)
    assert L["words"] == 6 * 256 * 64 == 98304
    assert L["word_bytes"] == 4 * 98304
    dense = 1024 * 4096 * 2
    assert dense / (4 * 16 * 256 * 64) == 8.0          # packing alone, all 16 tiles
    assert L["scale_bytes"] == 6 * 16 * 64 * 4
    assert L["total_bytes"] == L["word_bytes"] + L["scale_bytes"] + 4096 * 2 + 6 * 64 * 4


# ------------------------------------------------- compact code (the bundles' lengths)

def _compact_ok(lens):
    used = sorted(set(int(x) for x in lens if x))
    return len(used) <= 4 and max(used) <= 11 and all(L <= 8 for L in used[:-1]) and kraft_sum(lens) <= 2048


def _golden_rows(prefix):
    out = {}
    with open(os.path.join(GOLDEN, "canonical_small.txt")) as f:
        for line in f:
            if line.startswith(prefix):
                k, *v = line.split()
                out[k] = [int(x) for x in v]
    return out


def test_compact_golden_hand_worked():
    """The hand-worked compact codes of tests/golden/canonical_small.txt: a
    tie between two codes, a histogram whose optimum needs five lengths, and
    a tie that the search order decides."""
    g = _golden_rows("compact")
    for ck, lk in (("compact_counts", "compact_lens"), ("compact6_counts", "compact6_lens"),
                   ("compact7_counts", "compact7_lens")):
        lens = O.compact_lengths(np.array(g[ck], np.uint64))
        assert lens.tolist() == g[lk], (ck, lens.tolist())


@pytest.mark.parametrize("seed", range(40))
def test_compact_is_cheapest_allowed_code_exhaustive(seed):
    """Exhaustive search over EVERY length vector (1..11 per symbol, 2..5
    symbols) with at most four distinct lengths, the three shorter <= 8, and
    Kraft sum <= 1: its least total equals the oracle's."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 6))
    counts = rng.integers(1, 60, size=n).astype(np.uint64)
    if seed % 4 == 0:
        counts = np.array([1 << int(k) for k in rng.integers(0, 12, size=n)], np.uint64)   # skewed
    lens = O.compact_lengths(counts)
    assert _compact_ok(lens)
    got = int((lens.astype(np.int64) * counts.astype(np.int64)).sum())
    best = None
    for v in itertools.product(range(1, 12), repeat=n):
        if not _compact_ok(v):
            continue
        c = int(sum(int(a) * int(b) for a, b in zip(v, counts)))
        best = c if best is None or c < best else best
    assert got == best


@pytest.mark.parametrize("seed", range(12))
def test_compact_versus_package_merge(seed):
    """Never cheaper than the optimal 11-bit-limited code (package-merge);
    exactly as cheap when that code already uses at most four lengths with
    the three shorter <= 8; every rank no longer than a rarer one."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 257))
    counts = rng.integers(0, 1000, size=256).astype(np.uint64)
    counts[rng.permutation(256)[n:]] = 0
    if counts.sum() == 0:
        counts[0] = 5
    lens = O.compact_lengths(counts)
    pm = O.package_merge(counts)
    cost = lambda L: int((L.astype(np.int64) * counts.astype(np.int64)).sum())
    assert _compact_ok(lens)
    assert cost(lens) >= cost(pm)
    if _compact_ok(pm):
        assert cost(lens) == cost(pm)
    nz = np.nonzero(counts)[0]
    order = sorted(nz, key=lambda s: (-int(counts[s]), s))
    assert all(lens[order[i]] <= lens[order[i + 1]] for i in range(len(order) - 1))


def test_compact_degenerate_alphabets():
    assert O.compact_lengths(np.array([0, 7, 0], np.uint64)).tolist() == [0, 1, 0]
    assert O.compact_lengths(np.array([3, 9], np.uint64)).tolist() == [1, 1]
    assert set(O.compact_lengths(np.ones(256, np.uint64)).tolist()) == {8}
    assert set(O.compact_lengths(np.ones(16, np.uint64)).tolist()) == {4}


def test_compact_bits_on_workload_distribution():
    """4-bit pair symbols of q = clamp(rint(N(7.5, 1.8)), 0, 15), with counts
    proportional to the exact discretised distribution: 5.9419 bits per pair
    for the optimal 11-bit-limited code and 5.9775 for the compact one with
    lengths 5, 6, 8 and 11 (both figures from a separate dynamic program over
    length sets and splits, not from either implementation here)."""
    from math import erf, sqrt
    cdf = lambda t: 0.5 * (1.0 + erf((t - 7.5) / (1.8 * sqrt(2.0))))
    p = np.array([(1.0 if q == 15 else cdf(q + 0.5)) - (0.0 if q == 0 else cdf(q - 0.5)) for q in range(16)])
    pair = np.outer(p, p).ravel()                      # symbol = q_even | q_odd << 4
    counts = np.maximum(np.rint(pair * 1e12), 1).astype(np.uint64)
    w = counts.astype(np.float64) / counts.sum()
    lens = O.compact_lengths(counts)
    pm = O.package_merge(counts)
    assert abs(float((lens * w).sum()) - 5.9775) < 5e-4
    assert abs(float((pm * w).sum()) - 5.9419) < 5e-4
    assert sorted(set(lens.tolist())) == [5, 6, 8, 11]
