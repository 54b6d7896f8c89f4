"""ctypes binding of the C oracle (oracle.c) and the bundle pipeline built from it.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.  It shares no code
with the product (decode_gemv_amd) and never imports it.

The functions below chain the oracle's C steps in the order the method runs
them ("LazyWeights", section "2 . Code them" for the bundle, section "3 . Decode
on demand" for the decoder; "Unweight", exponent palette and verbatim rows for
bf16), using numpy only to hold arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

Q4, Q6, BF16 = 1, 2, 3
KIND = {"q4": Q4, "q6": Q6, "bf16": BF16}
MAXLEN = 11


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC",
                               "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(LIB)
        P = C.c_void_p
        i64, i32, u32 = C.c_int64, C.c_int, C.c_uint32
        sig = {
            "or_symbols_per_lane": (i32, [i32]),
            "or_alphabet": (i32, [i32]),
            "or_symbolise_q": (None, [i32, i64, i64, P, P]),
            "or_unsymbolise_q": (None, [i32, i64, i64, P, P]),
            "or_histogram": (None, [P, i64, i32, P]),
            "or_package_merge": (i32, [i32, P, i32, P]),
            "or_compact_lengths": (i32, [i32, P, P]),
            "or_rans_freqs": (i32, [i32, P, P, P]),
            "or_rans_symbolise": (None, [i32, i64, i64, P, P]),
            "or_rans_encode_tiles": (i64, [i64, i32, i32, P, P, P, P, P]),
            "or_rans_decode_tiles": (i32, [i64, i32, i32, i32, P, P, P, P, P]),
            "or_rans_encode_stream": (i32, [P, i32, P, P, P, P]),
            "or_rans_decode_stream": (i32, [u32, P, i64, i64, i32, i32, P, P, P]),
            "or_canonical": (i32, [i32, P, P, P, P, P, P, P]),
            "or_encode_tiles": (i64, [i64, i32, P, P, P, P, P, P]),
            "or_decode_limit": (i32, [i64, i32, P, P, P, P, P, P, P, P, P]),
            "or_decode_bitwise": (i32, [i64, i32, P, P, i32, P, P, P]),
            "or_half_to_double": (C.c_double, [C.c_uint16]),
            "or_double_to_half": (C.c_uint16, [C.c_double]),
            "or_swiglu": (None, [i64, P, P, P]),
            "or_bf16_to_double": (C.c_double, [C.c_uint16]),
            "or_pack_dm": (None, [i64, i64, P, P, P]),
            "or_gemv_q": (None, [i64, i64, P, P, P, P, i32, P, i64, P]),
            "or_gemv_bf16": (None, [i64, i64, P, P, i32, P, i64, P]),
            "or_bf16_palette": (i32, [i64, P, P]),
            "or_bf16_verbatim": (i64, [i64, i64, P, P, i32, P, P, P]),
            "or_bf16_symbolise": (None, [i64, i64, P, P, i32, P, P]),
            "or_bf16_pack_sm": (None, [i64, i64, P, P]),
            "or_bf16_reconstruct": (None, [i64, i64, P, P, P, P, P, P, P]),
            "or_skip_pack": (None, [i64, i64, i32, P, P, P, P, P]),
            "or_skip_gemv": (None, [i64, i64, i32, P, P, P, i64, P, i32, P]),
            "or_skip_ledger": (None, [i64, i32, i64, i32, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- steps

def symbols_per_lane(kind: int) -> int:
    return lib().or_symbols_per_lane(kind)


def alphabet(kind: int) -> int:
    return lib().or_alphabet(kind)


def symbolise_q(kind: int, codes: np.ndarray) -> np.ndarray:
    R, Cc = codes.shape
    nt = (R // 64) * (Cc // 256)
    syms = np.empty(nt * 32 * symbols_per_lane(kind), dtype=np.uint16)
    lib().or_symbolise_q(kind, R, Cc, _p(np.ascontiguousarray(codes, np.uint8)), _p(syms))
    return syms


def unsymbolise_q(kind: int, rows: int, cols: int, syms: np.ndarray) -> np.ndarray:
    q = np.empty((rows, cols), dtype=np.uint8)
    lib().or_unsymbolise_q(kind, rows, cols, _p(syms), _p(q))
    return q


def histogram(syms: np.ndarray, n_alpha: int) -> np.ndarray:
    counts = np.zeros(n_alpha, dtype=np.uint64)
    lib().or_histogram(_p(syms), syms.size, n_alpha, _p(counts))
    return counts


def package_merge(counts, limit: int = MAXLEN) -> np.ndarray:
    counts = np.ascontiguousarray(counts, dtype=np.uint64)
    lens = np.zeros(counts.size, dtype=np.uint8)
    rc = lib().or_package_merge(counts.size, _p(counts), limit, _p(lens))
    if rc != 0:
        raise ValueError("alphabet does not fit the length limit")
    return lens


def compact_lengths(counts) -> np.ndarray:
    """Lengths of the opt-in compact code: the cheapest prefix code with
    lengths <= 11 using at most four distinct lengths, the three shorter <= 8."""
    counts = np.ascontiguousarray(counts, dtype=np.uint64)
    lens = np.zeros(counts.size, dtype=np.uint8)
    if lib().or_compact_lengths(counts.size, _p(counts), _p(lens)) != 0:
        raise ValueError("more than 256 symbols")
    return lens


def canonical(lens: np.ndarray) -> dict:
    lens = np.ascontiguousarray(lens, dtype=np.uint8)
    n = lens.size
    codes = np.zeros(n, dtype=np.uint16)
    arr = {k: np.zeros(MAXLEN + 1, dtype=np.uint16) for k in ("count", "first", "limit", "offset")}
    sym_sorted = np.zeros(max(n, 1), dtype=np.uint16)
    k = lib().or_canonical(n, _p(lens), _p(codes), _p(arr["count"]), _p(arr["first"]),
                           _p(arr["limit"]), _p(arr["offset"]), _p(sym_sorted))
    if k < 0:
        raise ValueError("code length above 11")
    arr.update(codes=codes, lens=lens, sym_sorted=sym_sorted[:k].copy(), n_sym=k)
    return arr


def encode_tiles(syms: np.ndarray, spl: int, lens: np.ndarray, codes: np.ndarray):
    """-> (tile_off uint32 [T+1], words uint32, lane_bits uint32 [T*32])."""
    nt = syms.size // (32 * spl)
    tile_off = np.zeros(nt + 1, dtype=np.uint32)
    lane_bits = np.zeros(nt * 32, dtype=np.uint32)
    total = lib().or_encode_tiles(nt, spl, _p(syms), _p(lens), _p(codes), _p(tile_off), None,
                                  _p(lane_bits))
    words = np.zeros(max(total, 1), dtype=np.uint32)
    lib().or_encode_tiles(nt, spl, _p(syms), _p(lens), _p(codes), _p(tile_off), _p(words),
                          _p(lane_bits))
    return tile_off, words[:total], lane_bits


def decode_limit(tab: dict, tile_off, words, spl: int):
    """-> (syms, lane_bits) by the limit method."""
    nt = tile_off.size - 1
    out = np.zeros(nt * 32 * spl, dtype=np.uint16)
    bits = np.zeros(nt * 32, dtype=np.uint32)
    w = words if words.size else np.zeros(1, np.uint32)
    rc = lib().or_decode_limit(nt, spl, _p(tile_off), _p(w), _p(tab["count"]), _p(tab["first"]),
                               _p(tab["limit"]), _p(tab["offset"]), _p(tab["sym_sorted"]),
                               _p(out), _p(bits))
    if rc != 0:
        raise ValueError("peek matched no code length")
    return out, bits


def decode_bitwise(tab: dict, tile_off, words, spl: int):
    nt = tile_off.size - 1
    out = np.zeros(nt * 32 * spl, dtype=np.uint16)
    w = words if words.size else np.zeros(1, np.uint32)
    rc = lib().or_decode_bitwise(nt, spl, _p(tile_off), _p(w), tab["lens"].size,
                                 _p(tab["lens"]), _p(tab["codes"]), _p(out))
    if rc != 0:
        raise ValueError("bitwise decode ran past 11 bits")
    return out


def pack_dm(d: np.ndarray, m: np.ndarray) -> np.ndarray:
    R, ncb = d.shape
    dm = np.zeros(R * ncb, dtype=np.uint32)
    lib().or_pack_dm(R, ncb * 256, _p(np.ascontiguousarray(d, np.uint16)),
                     _p(np.ascontiguousarray(m, np.uint16)), _p(dm))
    return dm


def double_to_half(v: float) -> int:
    return lib().or_double_to_half(v)


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """fp16 bits of silu(g) * u, elementwise, from fp64 g and u."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    h = np.zeros(g.shape, dtype=np.uint16)
    lib().or_swiglu(g.size, _p(g), _p(u), _p(h))
    return h


def mlp_pass_q(gate, up, down, x, batch: int) -> np.ndarray:
    """One SwiGLU MLP pass over quantised matrices, all in fp64: gate, up and
    down are (codes, d, m) with down's columns = gate's rows; the gate and up
    outputs meet in swiglu (rounded to fp16 once), which is down's input.
    Returns y [batch][down rows]."""
    g = gemv_q(*gate, x, batch)
    u = gemv_q(*up, x, batch)
    return gemv_q(*down, swiglu(g, u), batch)


def gemv_q(codes, d, m, x, batch: int, rows=None) -> np.ndarray:
    """fp64 y [batch][len(rows) or R] from codes, fp16 d/m and fp16 x bits."""
    R, Cc = codes.shape
    x = np.ascontiguousarray(x[:batch], dtype=np.uint16)
    rl = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = R if rl is None else rl.size
    y = np.zeros((batch, nr), dtype=np.float64)
    lib().or_gemv_q(R, Cc, _p(np.ascontiguousarray(codes, np.uint8)),
                    _p(np.ascontiguousarray(d, np.uint16)), _p(np.ascontiguousarray(m, np.uint16)),
                    _p(x), batch, _p(rl), nr, _p(y))
    return y


def gemv_bf16(w, x, batch: int, rows=None) -> np.ndarray:
    R, Cc = w.shape
    x = np.ascontiguousarray(x[:batch], dtype=np.uint16)
    rl = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = R if rl is None else rl.size
    y = np.zeros((batch, nr), dtype=np.float64)
    lib().or_gemv_bf16(R, Cc, _p(np.ascontiguousarray(w, np.uint16)), _p(x), batch, _p(rl), nr,
                       _p(y))
    return y


def half_to_double(h: int) -> float:
    return lib().or_half_to_double(h)


def bf16_to_double(b: int) -> float:
    return lib().or_bf16_to_double(b)


# ---------------------------------------------------------------- bundles

def row_split(syms: np.ndarray, spl: int, lens: np.ndarray) -> np.ndarray:
    """Per tile and lane, the number of bits of the lane's first tile row
    (its first spl/2 symbols): the bit of the lane stream where its second
    row starts.  u16 [n_tiles * 32]."""
    s = np.asarray(syms).reshape(-1, 32, spl)[:, :, :spl // 2]
    return np.asarray(lens, dtype=np.int64)[s].sum(axis=2).astype(np.uint16).ravel()


# Decoding units (tiles x parts per tile row) the default part count stays within.
PART_UNITS = 4096


def default_parts(n_tiles: int, n_cb: int = 0, quantised: bool = False) -> int:
    """Parts per tile row when the caller leaves it open: the largest of 8, 4,
    2 that keeps n_tiles * parts <= PART_UNITS, else 1; for 4- and 6-bit
    codes 2 also where n_tiles is an odd multiple of 512 in (PART_UNITS / 2,
    PART_UNITS] and a row band has more than 16 column blocks (n_cb)."""
    for p in (8, 4, 2):
        if n_tiles * p <= PART_UNITS:
            return p
    if quantised and PART_UNITS // 2 < n_tiles <= PART_UNITS and n_tiles % 512 == 0 and (n_tiles // 512) % 2 == 1 \
            and n_cb > 16:
        return 2
    return 1


def part_starts(syms: np.ndarray, spl: int, lens: np.ndarray, parts: int) -> np.ndarray:
    """Each lane stream cut into 2*parts runs of spl/(2*parts) symbols (parts
    per tile row): for k = 1 .. 2*parts-1, the bit where run k begins (the
    total length of the runs before it).  u16 [n_tiles][2*parts-1][32]; with
    parts = 1 this is row_split."""
    s = np.asarray(syms).reshape(-1, 32, spl)
    L = np.asarray(lens, dtype=np.int64)[s]                     # [tiles][lane][symbol]
    per = spl // (2 * parts)
    ends = np.cumsum(L, axis=2)[:, :, per - 1::per]             # bits through the end of each run
    starts = ends[:, :, :2 * parts - 1]                         # run k starts where run k-1 ends
    return starts.transpose(0, 2, 1).astype(np.uint16).ravel()


def code_lengths(counts, code: str = "huffman") -> np.ndarray:
    """The bundle's code lengths: "huffman" (the default) is the optimal
    prefix code with lengths <= 11, the length-limited Huffman table of
    "LazyWeights", section "2 . Code them", found by package-merge;
    "compact" is the opt-in code with at most four lengths."""
    if code == "huffman":
        return package_merge(counts)
    if code == "compact":
        return compact_lengths(counts)
    raise ValueError(f"unknown code {code!r}")


def build_bundle_q(kind: int, codes: np.ndarray, d: np.ndarray, m: np.ndarray, code: str = "huffman",
                   lens=None, parts: int = 0) -> dict:
    """Quantised bundle: per-matrix table, tile offsets, interleaved words, dm,
    part starts.  `lens` (one length per symbol), when given, replaces the
    chosen code's; parts 0 takes default_parts."""
    R, Cc = codes.shape
    if R % 64 or Cc % 256:
        raise ValueError("shape must be a multiple of 64x256")
    spl = symbols_per_lane(kind)
    syms = symbolise_q(kind, codes)
    counts = histogram(syms, alphabet(kind))
    lens = code_lengths(counts, code) if lens is None else np.ascontiguousarray(lens, dtype=np.uint8)
    tab = canonical(lens)
    tile_off, words, lane_bits = encode_tiles(syms, spl, lens, tab["codes"])
    parts = parts or default_parts((R // 64) * (Cc // 256), Cc // 256, quantised=True)
    return dict(kind=kind, rows=R, cols=Cc, spl=spl, counts=counts, table=tab,
                tile_off=tile_off, words=words, lane_bits=lane_bits, dm=pack_dm(d, m),
                parts=parts, split=part_starts(syms, spl, lens, parts))


def decode_bundle_q(b: dict, bitwise: bool = False):
    """-> (codes [R][C], lane_bits or None)."""
    if bitwise:
        syms, bits = decode_bitwise(b["table"], b["tile_off"], b["words"], b["spl"]), None
    else:
        syms, bits = decode_limit(b["table"], b["tile_off"], b["words"], b["spl"])
    return unsymbolise_q(b["kind"], b["rows"], b["cols"], syms), bits


def symbolise_bf16(w: np.ndarray, palette: np.ndarray, n_pal: int, vb_bits: np.ndarray) -> np.ndarray:
    """Lane symbol streams of a bf16 matrix: palette indices, placeholder 0
    inside verbatim segments; u16 [n_tiles * 32 * 512]."""
    R, Cc = w.shape
    w = np.ascontiguousarray(w, dtype=np.uint16)
    syms = np.zeros((R // 64) * (Cc // 256) * 32 * 512, dtype=np.uint16)
    lib().or_bf16_symbolise(R, Cc, _p(w), _p(np.ascontiguousarray(palette)), n_pal,
                            _p(np.ascontiguousarray(vb_bits)), _p(syms))
    return syms


def build_bundle_bf16(w: np.ndarray, code: str = "huffman", parts: int = 0) -> dict:
    R, Cc = w.shape
    if R % 64 or Cc % 256:
        raise ValueError("shape must be a multiple of 64x256")
    w = np.ascontiguousarray(w, dtype=np.uint16)
    L = lib()
    palette = np.zeros(16, dtype=np.uint8)
    n_pal = L.or_bf16_palette(w.size, _p(w), _p(palette))
    nt = (R // 64) * (Cc // 256)
    vb_bits = np.zeros(nt * 8, dtype=np.uint32)
    vb_start = np.zeros(nt + 1, dtype=np.uint32)
    nv = L.or_bf16_verbatim(R, Cc, _p(w), _p(palette), n_pal, _p(vb_bits), _p(vb_start), None)
    verbatim = np.zeros(max(nv, 1) * 64, dtype=np.uint16)
    L.or_bf16_verbatim(R, Cc, _p(w), _p(palette), n_pal, _p(vb_bits), _p(vb_start), _p(verbatim))
    syms = symbolise_bf16(w, palette, n_pal, vb_bits)
    counts = histogram(syms, 16)
    lens = code_lengths(counts, code)
    tab = canonical(lens)
    tile_off, words, lane_bits = encode_tiles(syms, 512, lens, tab["codes"])
    sm = np.zeros(nt * 4096, dtype=np.uint32)
    L.or_bf16_pack_sm(R, Cc, _p(w), _p(sm))
    return dict(kind=BF16, rows=R, cols=Cc, spl=512, counts=counts, table=tab, palette=palette,
                n_pal=n_pal, vb_bits=vb_bits, vb_start=vb_start, verbatim=verbatim[:nv * 64],
                n_verbatim=nv, tile_off=tile_off, words=words, lane_bits=lane_bits, sm=sm,
                parts=parts or default_parts(nt), split=part_starts(syms, 512, lens, parts or default_parts(nt)))


def decode_bundle_bf16(b: dict, bitwise: bool = False):
    if bitwise:
        syms, bits = decode_bitwise(b["table"], b["tile_off"], b["words"], 512), None
    else:
        syms, bits = decode_limit(b["table"], b["tile_off"], b["words"], 512)
    R, Cc = b["rows"], b["cols"]
    out = np.zeros((R, Cc), dtype=np.uint16)
    verb = b["verbatim"] if b["verbatim"].size else np.zeros(64, np.uint16)
    lib().or_bf16_reconstruct(R, Cc, _p(syms), _p(b["sm"]), _p(b["palette"]), _p(b["vb_bits"]),
                              _p(b["vb_start"]), _p(verb), _p(out))
    return out, bits


# ---------------------------------------------------------------- tile-skipping twin
SKIP_BN = 64


def skip_pack(codes: np.ndarray, bits: int, d: np.ndarray, m: np.ndarray):
    """Tile-transposed fixed-width words [tiles][WPR][64] and scales
    [tiles][cols/256][64] ("Software-Defined Bandwidth Expansion" IV-A, IV-B)."""
    R, Cc = codes.shape
    wpr = Cc // (32 // bits)
    words = np.zeros((R // SKIP_BN) * wpr * SKIP_BN, dtype=np.uint32)
    dm = np.zeros((R // SKIP_BN) * (Cc // 256) * SKIP_BN, dtype=np.uint32)
    lib().or_skip_pack(R, Cc, bits, _p(np.ascontiguousarray(codes, np.uint8)),
                       _p(np.ascontiguousarray(d, np.uint16)), _p(np.ascontiguousarray(m, np.uint16)),
                       _p(words), _p(dm))
    return words, dm


def skip_gemv(words, dm, bits: int, rows: int, cols: int, tiles, x, batch: int, y=None) -> np.ndarray:
    """fp64 y [batch][rows]: rows of listed tiles computed from the packed
    words, every other row left as it was in y (NaN when y is not given)."""
    tl = np.ascontiguousarray(tiles, dtype=np.int32)
    x = np.ascontiguousarray(x[:batch], dtype=np.uint16)
    if y is None:
        y = np.full((batch, rows), np.nan)
    lib().or_skip_gemv(rows, cols, bits, _p(words), _p(dm), _p(tl) if tl.size else None, tl.size, _p(x),
                       batch, _p(y))
    return y


def skip_ledger(cols: int, bits: int, n_active: int, batch: int) -> dict:
    out = np.zeros(6, dtype=np.uint64)
    lib().or_skip_ledger(cols, bits, n_active, batch, _p(out))
    return dict(zip(("words", "word_bytes", "scale_bytes", "x_bytes", "y_bytes", "total_bytes"),
                    (int(v) for v in out)))


# ---------------------------------------------------------------- rANS lane coder (ablation)
RANS_M = 2048
RANS_L = 1 << 16


def rans_freqs(counts) -> tuple:
    counts = np.ascontiguousarray(counts, dtype=np.uint64)
    f = np.zeros(counts.size, dtype=np.uint16)
    cum = np.zeros(counts.size, dtype=np.uint16)
    if lib().or_rans_freqs(counts.size, _p(counts), _p(f), _p(cum)) < 0:
        raise ValueError("frequencies do not fit")
    return f, cum


def rans_symbolise(kind: int, codes: np.ndarray) -> np.ndarray:
    R, Cc = codes.shape
    spr = 128 if kind == Q4 else 256
    syms = np.empty((R // 64) * (Cc // 256) * 64 * spr, dtype=np.uint16)
    lib().or_rans_symbolise(kind, R, Cc, _p(np.ascontiguousarray(codes, np.uint8)), _p(syms))
    return syms


def rans_encode_stream(syms, f, cum) -> tuple:
    """One stream: (final encoder state, 16-bit chunks in decoding order)."""
    syms = np.ascontiguousarray(syms, np.uint16)
    f = np.ascontiguousarray(f, np.uint16)
    cum = np.ascontiguousarray(cum, np.uint16)
    st = np.zeros(1, np.uint32)
    ch = np.zeros(max(syms.size, 1), np.uint16)
    k = lib().or_rans_encode_stream(_p(syms), syms.size, _p(f), _p(cum), _p(st), _p(ch))
    return int(st[0]), ch[:k].copy()


def rans_decode_stream(state, chunks, n, f, cum) -> np.ndarray:
    """n symbols of one stream (consecutive chunks), or ValueError."""
    chunks = np.ascontiguousarray(chunks, np.uint16)
    if chunks.size == 0:
        chunks = np.zeros(1, np.uint16)
        nch = 0
    else:
        nch = chunks.size
    f = np.ascontiguousarray(f, np.uint16)
    cum = np.ascontiguousarray(cum, np.uint16)
    out = np.zeros(max(n, 1), np.uint16)
    if lib().or_rans_decode_stream(state, _p(chunks), 1, nch, n, f.size, _p(f), _p(cum), _p(out)) != 0:
        raise ValueError("rANS stream does not decode to its final state")
    return out[:n]


def build_rans_q(kind: int, codes: np.ndarray, halves: int = 1) -> dict:
    """rANS bundle content: frequencies, cumulative frequencies, tile offsets,
    words, and the streams' symbols [t][ns][sps] (ns = 64 * halves streams a
    tile, sps symbols a stream; with two halves, stream h*64 + r is half h of
    row r)."""
    R, Cc = codes.shape
    spr = 128 if kind == Q4 else 256
    nt = (R // 64) * (Cc // 256)
    rows = rans_symbolise(kind, codes)                                   # [t][64][spr]
    sps = spr // halves
    syms = np.ascontiguousarray(rows.reshape(nt, 64, halves, sps).transpose(0, 2, 1, 3)).reshape(-1)
    counts = histogram(syms, alphabet(kind))
    f, cum = rans_freqs(counts)
    ns = 64 * halves
    tile_off = np.zeros(nt + 1, dtype=np.uint32)
    n = lib().or_rans_encode_tiles(nt, ns, sps, _p(syms), _p(f), _p(cum), _p(tile_off), None)
    words = np.zeros(max(n, 1), dtype=np.uint32)
    lib().or_rans_encode_tiles(nt, ns, sps, _p(syms), _p(f), _p(cum), _p(tile_off), _p(words))
    return dict(kind=kind, rows=R, cols=Cc, spr=spr, halves=halves, ns=ns, sps=sps, counts=counts, f=f, cum=cum,
                tile_off=tile_off, words=words[:n], syms=syms)


def decode_rans(b: dict) -> np.ndarray:
    """Symbols of every stream ([t][ns][sps]), or ValueError for a stream that does not end in state L."""
    nt = b["tile_off"].size - 1
    syms = np.zeros(nt * b["ns"] * b["sps"], dtype=np.uint16)
    w = b["words"] if b["words"].size else np.zeros(1, np.uint32)
    rc = lib().or_rans_decode_tiles(nt, b["ns"], b["sps"], b["f"].size, _p(b["f"]), _p(b["cum"]), _p(b["tile_off"]),
                                    _p(w), _p(syms))
    if rc != 0:
        raise ValueError("rANS stream does not decode to its final state")
    return syms


def rans_unsymbolise(kind: int, rows: int, cols: int, syms: np.ndarray, halves: int = 1) -> np.ndarray:
    """Codes [rows][cols] from the stream symbols [t][ns][sps] (numpy; inverse of build_rans_q's layout)."""
    spr = 128 if kind == Q4 else 256
    nt = (rows // 64) * (cols // 256)
    s = np.asarray(syms).reshape(nt, halves, 64, spr // halves).transpose(0, 2, 1, 3)
    s = s.reshape(rows // 64, cols // 256, 64, spr)
    if kind == Q4:
        q = np.empty((rows // 64, cols // 256, 64, 256), dtype=np.uint8)
        q[..., 0::2] = s & 15
        q[..., 1::2] = s >> 4
    else:
        q = s.astype(np.uint8)
    return q.transpose(0, 2, 1, 3).reshape(rows, cols)


# ---------------------------------------------------------------- bf16 compact forms (reconstructive GEMM)
def transcode_forms(b: dict, w: np.ndarray) -> dict:
    """The compact forms of a bf16 matrix that the reconstructive GEMM reads
    ("Unweight", "Four approaches to using compressed weights"), from the
    oracle's palette and verbatim map (numpy):
      palette : u32 [t][32][64], 8 palette indices of columns 8g..8g+7 of tile
                row r, the lowest column in the low nibble
      exponent: u32 [t][64][64], 4 exponent bytes of columns 4g..4g+3
      vrank   : i32 [t][4][64], the verbatim store index of segment s of tile
                row r (tiles in order, then rows, then segments), or -1
    Weights of a verbatim segment carry palette index 0 (the placeholder)."""
    R, Cc = w.shape
    nrb, ncb = R // 64, Cc // 256
    pal = b["palette"][:b["n_pal"]]
    idx_of = np.full(256, -1, dtype=np.int64)
    idx_of[pal] = np.arange(pal.size)
    idx = idx_of[(w.astype(np.int64) >> 7) & 0xFF]                       # [R][C]
    bits = np.unpackbits(b["vb_bits"].view(np.uint8), bitorder="little").reshape(nrb, ncb, 64, 4)  # [rb][cb][i][s]
    verb = bits.transpose(0, 2, 1, 3).reshape(R, Cc // 64).astype(bool)   # [row][64-column segment]
    idx[np.repeat(verb, 64, axis=1)] = 0
    if np.any(idx < 0):
        raise ValueError("an exponent outside the palette lies outside every verbatim segment")
    I = idx.reshape(nrb, 64, ncb, 32, 8)
    palw = (I << (4 * np.arange(8))).sum(-1).astype(np.uint32)         # [rb][i][cb][g]
    E = b["palette"][idx].astype(np.int64).reshape(nrb, 64, ncb, 64, 4)
    expw = (E << (8 * np.arange(4))).sum(-1).astype(np.uint32)
    # rank of each set bit of a tile's map, in map order, offset by the tile's start
    flat = bits.reshape(nrb * ncb, 256)
    rank = np.cumsum(flat, axis=1) - flat + b["vb_start"][:-1, None].astype(np.int64)
    vr = np.where(flat == 1, rank, -1).reshape(nrb * ncb, 64, 4).transpose(0, 2, 1)   # [t][s][i]
    return dict(palette=palw.transpose(0, 2, 3, 1).reshape(-1), exponent=expw.transpose(0, 2, 3, 1).reshape(-1),
                vrank=vr.astype(np.int32).reshape(-1))


def rebuild_from_form(b: dict, forms: dict, form: str, rows: int, cols: int) -> np.ndarray:
    """bf16 weights [rows][cols] rebuilt from a compact form, the sign+mantissa
    stream and the verbatim store (numpy; the check that a form is complete)."""
    nrb, ncb = rows // 64, cols // 256
    if form == "palette":
        wv = forms["palette"].reshape(nrb, ncb, 32, 64).astype(np.int64)
        nib = (wv[..., None] >> (4 * np.arange(8))) & 15                  # [rb][cb][g][i][j]
        e = b["palette"][nib.transpose(0, 3, 1, 2, 4).reshape(rows, cols)].astype(np.int64)
    else:
        wv = forms["exponent"].reshape(nrb, ncb, 64, 64).astype(np.int64)
        by = (wv[..., None] >> (8 * np.arange(4))) & 255
        e = by.transpose(0, 3, 1, 2, 4).reshape(rows, cols)
    smw = b["sm"].reshape(nrb, ncb, 2, 64, 32).astype(np.int64)           # [rb][cb][i&1][g4][i>>1]
    smb = (smw[..., None] >> (8 * np.arange(4))) & 255                     # [..][g4][i>>1][j]
    smb = smb.transpose(0, 4, 2, 1, 3, 5).reshape(nrb, 64, ncb, 256)      # [rb][i>>1][i&1][cb][g4 j]
    sm = smb.reshape(rows, cols)
    out = ((sm >> 7) << 15) | (e << 7) | (sm & 0x7F)
    vr = forms["vrank"].reshape(nrb, ncb, 4, 64)
    for rb, cb, s, i in zip(*np.nonzero(vr >= 0)):
        v = int(vr[rb, cb, s, i])
        r, c0 = 64 * rb + i, 256 * cb + 64 * s
        out[r, c0:c0 + 64] = b["verbatim"][64 * v:64 * v + 64]
    return out.astype(np.uint16)
