"""CPU tests of the product's host side: the C ABI loads and exports what
include/lw.h declares, the bundle builder produces exactly the oracle's
format, and validation rejects corrupt images.  No GPU call is made."""
import ctypes

import numpy as np
import pytest

import decode_gemv_amd as dg
import oracle as O
import synth


def test_library_exports_every_declared_symbol():
    names = dg.header_functions()
    assert len(names) >= 16
    lib = ctypes.CDLL(dg.lw.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _table_from_region(b):
    t = dg.lw_bundle_region(b, dg.LW_REG_TABLE, np.uint16)
    return dict(count=t[0:12], first=t[12:24], limit=t[24:36], offset=t[36:48], sym_sorted=t[48:])


def _compare_q(kind, codes, d, m, code="huffman"):
    ob = O.build_bundle_q(kind, codes, d, m, code=code)
    build = dg.lw_bundle_build_q if code == "huffman" else dg.lw_bundle_build_q_compact
    pb = build(kind, codes, d, m)
    dg.lw_bundle_validate(pb)
    info = dg.lw_bundle_get_info(pb)
    assert info["code"] == (dg.LW_CODE_HUFFMAN if code == "huffman" else dg.LW_CODE_COMPACT)
    tab = _table_from_region(pb)
    for k in ("count", "first", "limit", "offset"):
        assert np.array_equal(tab[k], ob["table"][k]), k
    n = ob["table"]["n_sym"]
    assert info["n_symbols"] == n
    assert np.array_equal(tab["sym_sorted"][:n], ob["table"]["sym_sorted"])
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_TILE_OFF, np.uint32), ob["tile_off"])
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_WORDS, np.uint32), ob["words"])
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_DM, np.uint32), ob["dm"])
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_SPLIT, np.uint16), ob["split"])
    assert info["parts"] == ob["parts"] == O.default_parts(info["n_tiles"], codes.shape[1] // 256, quantised=True)
    W = np.diff(ob["tile_off"].astype(np.int64)) // 32
    assert info["max_words"] == W.max()
    assert info["coded_bytes"] == (ob["words"].nbytes + ob["tile_off"].nbytes + ob["dm"].nbytes +
                                   ob["split"].nbytes + 608)
    return pb, ob, info


@pytest.mark.parametrize("kind,rows,cols,law,seed", [
    (dg.LW_Q4_PAIR, 64, 256, "normal", 1), (dg.LW_Q4_PAIR, 192, 1024, "normal", 2),
    (dg.LW_Q4_PAIR, 128, 768, "laplace", 3), (dg.LW_Q6_SINGLE, 128, 512, "normal", 4),
    (dg.LW_Q4_PAIR, 64, 512, "uniform", 5), (dg.LW_Q4_PAIR, 64, 256, "const", 6),
    (dg.LW_Q6_SINGLE, 64, 256, "uniform", 7), (dg.LW_Q6_SINGLE, 64, 256, "const", 8)])
@pytest.mark.parametrize("code", ["huffman", "compact"])
def test_builder_matches_oracle_bytes(kind, rows, cols, law, seed, code):
    qmax = 15 if kind == dg.LW_Q4_PAIR else 63
    codes, d, m, _ = synth.gen_q_custom(rows, cols, seed, qmax=qmax, law=law,
                                        mu=7.5 if qmax == 15 else 31.5, scale=1.8 if qmax == 15 else 5.0)
    _compare_q(kind, codes, d, m, code)


@pytest.mark.parametrize("kind,law,seed", [(dg.LW_Q4_PAIR, "normal", 41), (dg.LW_Q4_PAIR, "laplace", 42),
                                            (dg.LW_Q6_SINGLE, "normal", 43)])
def test_builder_with_given_lengths_matches_oracle(kind, law, seed):
    """Caller-chosen code lengths (here the optimal 11-bit-limited code by
    package-merge, which uses more than four lengths: the decoders' general
    plan) give the oracle's canonical table, tile offsets, words and splits."""
    qmax = 15 if kind == dg.LW_Q4_PAIR else 63
    codes, d, m, _ = synth.gen_q_custom(192, 1280, seed, qmax=qmax, law=law,
                                        mu=7.5 if qmax == 15 else 31.5, scale=1.8 if qmax == 15 else 5.0)
    ok = O.Q4 if kind == dg.LW_Q4_PAIR else O.Q6
    syms = O.symbolise_q(ok, codes)
    lens = O.package_merge(O.histogram(syms, O.alphabet(ok)))
    assert len(set(lens[lens > 0].tolist())) > 4
    tab = O.canonical(lens)
    spl = O.symbols_per_lane(ok)
    tile_off, words, _ = O.encode_tiles(syms, spl, lens, tab["codes"])
    pb = dg.lw_bundle_build_q_lens(kind, codes, d, m, lens)
    dg.lw_bundle_validate(pb)
    t = _table_from_region(pb)
    for k in ("count", "first", "limit", "offset"):
        assert np.array_equal(t[k], tab[k]), k
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_TILE_OFF, np.uint32), tile_off)
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_WORDS, np.uint32), words)
    parts = O.default_parts((192 // 64) * (1280 // 256))
    assert dg.lw_bundle_get_info(pb)["parts"] == parts
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_SPLIT, np.uint16), O.part_starts(syms, spl, lens, parts))


@pytest.mark.parametrize("parts", [1, 2, 4, 8])
def test_builder_parts_match_oracle(parts):
    """Explicit parts per tile row: the part starts (and everything else)
    equal the oracle's for Q4, Q6 and bf16, with either code."""
    for kind, qmax, mu, sc in ((dg.LW_Q4_PAIR, 15, 7.5, 1.8), (dg.LW_Q6_SINGLE, 63, 31.5, 5.0)):
        codes, d, m, _ = synth.gen_q_custom(128, 768, 90 + parts, qmax=qmax, mu=mu, scale=sc)
        for code, cname in ((dg.LW_CODE_HUFFMAN, "huffman"), (dg.LW_CODE_COMPACT, "compact")):
            ob = O.build_bundle_q(kind, codes, d, m, code=cname, parts=parts)
            pb = dg.lw_bundle_build_q_opts(kind, codes, d, m, code=code, parts=parts)
            dg.lw_bundle_validate(pb)
            info = dg.lw_bundle_get_info(pb)
            assert info["parts"] == parts and info["code"] == code
            assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_WORDS, np.uint32), ob["words"])
            sp = dg.lw_bundle_region(pb, dg.LW_REG_SPLIT, np.uint16)
            assert sp.size == info["n_tiles"] * 32 * (2 * parts - 1)
            assert np.array_equal(sp, ob["split"])
            assert info["coded_bytes"] == (ob["words"].nbytes + ob["tile_off"].nbytes + ob["dm"].nbytes +
                                           ob["split"].nbytes + 608)
    w, _ = synth.gen_bf16_custom(128, 768, 95 + parts, outlier_frac=0.01)
    ob = O.build_bundle_bf16(w, parts=parts)
    pb = dg.lw_bundle_build_bf16_opts(w, parts=parts)
    assert dg.lw_bundle_get_info(pb)["parts"] == parts
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_SPLIT, np.uint16), ob["split"])
    # lengths given through the options match lw_bundle_build_q_lens
    codes, d, m, _ = synth.gen_q_custom(64, 512, 97)
    lens = O.package_merge(O.histogram(O.symbolise_q(O.Q4, codes), 256))
    a = dg.lw_bundle_build_q_opts(dg.LW_Q4_PAIR, codes, d, m, code=dg.LW_CODE_LENS, parts=parts, lens=lens)
    ob = O.build_bundle_q(O.Q4, codes, d, m, lens=lens, parts=parts)
    assert np.array_equal(dg.lw_bundle_region(a, dg.LW_REG_SPLIT, np.uint16), ob["split"])
    assert np.array_equal(dg.lw_bundle_region(a, dg.LW_REG_WORDS, np.uint32), ob["words"])


def test_build_options_rejected():
    codes, d, m, _ = synth.gen_q_custom(64, 256, 98)
    for parts in (3, 16, -1):
        with pytest.raises(dg.LwError) as e:
            dg.lw_bundle_build_q_opts(dg.LW_Q4_PAIR, codes, d, m, parts=parts)
        assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_build_q_opts(dg.LW_Q4_PAIR, codes, d, m, code=7)
    assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:               # LENS without lengths
        dg.lw_bundle_build_q_opts(dg.LW_Q4_PAIR, codes, d, m, code=dg.LW_CODE_LENS)
    assert e.value.status == dg.LW_E_ARG
    w, _ = synth.gen_bf16_custom(64, 256, 99)
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_build_bf16_opts(w, code=dg.LW_CODE_LENS)
    assert e.value.status == dg.LW_E_UNSUPPORTED


def test_given_lengths_rejected():
    codes, d, m, _ = synth.gen_q_custom(64, 256, 44)
    syms = O.symbolise_q(O.Q4, codes)
    lens = O.package_merge(O.histogram(syms, 256))
    missing = lens.copy()
    missing[np.flatnonzero(lens)[0]] = 0                  # a symbol that occurs without a length
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_build_q_lens(dg.LW_Q4_PAIR, codes, d, m, missing)
    assert e.value.status == dg.LW_E_TABLE
    with pytest.raises(dg.LwError) as e:                  # 256 codes of one bit: Kraft sum 128
        dg.lw_bundle_build_q_lens(dg.LW_Q4_PAIR, codes, d, m, np.ones(256, np.uint8))
    assert e.value.status == dg.LW_E_TABLE
    # a length above 11 is refused by the C side (called directly, as any C caller would) ...
    c12 = np.ascontiguousarray(codes, np.uint8)
    dd, mm = np.ascontiguousarray(d, np.uint16), np.ascontiguousarray(m, np.uint16)
    l12 = np.full(256, 12, np.uint8)
    out = ctypes.c_void_p()
    st = dg.lw.lib().lw_bundle_build_q_lens(dg.LW_Q4_PAIR, 64, 256, c12.ctypes.data, dd.ctypes.data,
                                            mm.ctypes.data, l12.ctypes.data, ctypes.byref(out))
    assert st == dg.LW_E_TABLE and not out.value
    # ... and by the binding before any byte cast could wrap it (267 would become 11)
    for bad in (np.full(256, 12, np.int32), np.full(256, 267, np.int64), np.full(256, -1, np.int16),
                np.full(256, 5.0)):
        with pytest.raises(ValueError):
            dg.lw_bundle_build_q_lens(dg.LW_Q4_PAIR, codes, d, m, bad)


@pytest.mark.parametrize("code", ["huffman", "compact"])
def test_builder_matches_oracle_workload_shapes(code):
    for wl in ("q4_256x1024", "q4_up_14336x4096", "q4_down_4096x14336", "q6_mlp_70b"):
        mat = synth.WORKLOADS[wl][0]
        kind = dg.LW_Q4_PAIR if mat.kind == "q4" else dg.LW_Q6_SINGLE
        codes, d, m, _ = synth.gen_q(mat, rows=min(mat.rows, 256), cols=min(mat.cols, 4096))
        _compare_q(kind, codes, d, m, code)


def test_default_code_is_the_optimal_length_limited_code():
    """The default bundle's table is package-merge's (the oracle's optimal
    11-bit-limited code): its total bits equal the oracle's, the compact
    option's are never fewer, and lengths 9 to 11 occur (the general
    comparison plan of the decoders is the one the default format needs)."""
    mat = synth.WORKLOADS["q4_up_14336x4096"][0]
    codes, d, m, _ = synth.gen_q(mat, rows=256, cols=4096)
    counts = O.histogram(O.symbolise_q(O.Q4, codes), 256)
    pm = O.package_merge(counts).astype(np.int64)
    huff = dg.lw_bundle_get_info(dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m))
    comp = dg.lw_bundle_get_info(dg.lw_bundle_build_q_compact(dg.LW_Q4_PAIR, codes, d, m))
    lens_h = np.repeat(np.arange(12), huff["count_per_len"])
    assert lens_h.size == np.count_nonzero(counts)
    assert sorted(lens_h.tolist()) == sorted(pm[counts > 0].tolist())
    assert huff["max_len"] == 11 and huff["min_len"] == 5
    assert comp["coded_bytes"] >= huff["coded_bytes"]
    assert huff["code"] == dg.LW_CODE_HUFFMAN and comp["code"] == dg.LW_CODE_COMPACT


@pytest.mark.parametrize("code", ["huffman", "compact"])
@pytest.mark.parametrize("frac,seed", [(0.0, 11), (0.002, 12), (0.02, 13)])
def test_builder_matches_oracle_bf16(frac, seed, code):
    w, _ = synth.gen_bf16_custom(128, 512, seed, outlier_frac=frac)
    ob = O.build_bundle_bf16(w, code=code)
    pb = (dg.lw_bundle_build_bf16 if code == "huffman" else dg.lw_bundle_build_bf16_compact)(w)
    dg.lw_bundle_validate(pb)
    info = dg.lw_bundle_get_info(pb)
    tab = _table_from_region(pb)
    for k in ("count", "first", "limit", "offset"):
        assert np.array_equal(tab[k], ob["table"][k]), k
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_PALETTE, np.uint8), ob["palette"])
    assert info["n_palette"] == ob["n_pal"] and info["n_verbatim"] == ob["n_verbatim"]
    for reg, key in ((dg.LW_REG_TILE_OFF, "tile_off"), (dg.LW_REG_WORDS, "words"), (dg.LW_REG_SM, "sm"),
                     (dg.LW_REG_VB_BITS, "vb_bits"), (dg.LW_REG_VB_START, "vb_start")):
        assert np.array_equal(dg.lw_bundle_region(pb, reg, np.uint32), ob[key]), key
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_VERBATIM, np.uint16), ob["verbatim"])
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_SPLIT, np.uint16), ob["split"])


def test_bf16_workload_shape_sample():
    w, _ = synth.gen_bf16(synth.WORKLOADS["bf16_up_14336x4096"][0], rows=256, cols=4096)
    ob = O.build_bundle_bf16(w)
    pb = dg.lw_bundle_build_bf16(w)
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_WORDS, np.uint32), ob["words"])
    assert np.array_equal(dg.lw_bundle_region(pb, dg.LW_REG_VERBATIM, np.uint16), ob["verbatim"])


def test_twin_layout():
    codes, d, m, _ = synth.gen_q_custom(64, 512, 21)
    twin, dm = dg.lw_twin_build(codes, 4, d, m)
    assert np.array_equal(twin & 15, codes[:, 0::2]) and np.array_equal(twin >> 4, codes[:, 1::2])
    assert np.array_equal(dm & 0xFFFF, d) and np.array_equal(dm >> 16, m)


# ------------------------------------------------------------------ errors

def test_argument_errors():
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_build_q(dg.LW_Q4_PAIR, np.zeros((65, 256), np.uint8), np.zeros((65, 1), np.uint16),
                             np.zeros((65, 1), np.uint16))
    assert e.value.status == dg.LW_E_SHAPE
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_build_q(dg.LW_Q4_PAIR, np.full((64, 256), 16, np.uint8), np.zeros((64, 1), np.uint16),
                             np.zeros((64, 1), np.uint16))
    assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_build_q(7, np.zeros((64, 256), np.uint8), np.zeros((64, 1), np.uint16),
                             np.zeros((64, 1), np.uint16))
    assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_build_bf16(np.zeros((64, 100), np.uint16))
    assert e.value.status == dg.LW_E_SHAPE
    assert dg.lw_status_str(dg.LW_E_TABLE) == "invalid code table"


def test_swiglu_argument_rules():
    # host-side checks only: each of these returns before any HIP call
    from decode_gemv_amd import lw
    assert lw._L.lw_swiglu(None, None, None, 0, None) == dg.LW_OK          # empty: nothing touched
    assert lw._L.lw_swiglu(None, None, None, -1, None) == dg.LW_E_ARG
    assert lw._L.lw_swiglu(None, None, None, 5, None) == dg.LW_E_ARG


def _image(seed=31, kind=dg.LW_Q4_PAIR):
    codes, d, m, _ = synth.gen_q_custom(128, 1024, seed)
    b = dg.lw_bundle_build_q(kind, codes, d, m)
    return b, dg.lw_bundle_image(b), dg.lw_bundle_get_info(b)


def test_load_round_trip():
    b, img, info = _image()
    b2 = dg.lw_bundle_load(img)
    assert np.array_equal(dg.lw_bundle_image(b2), img)


@pytest.mark.parametrize("what", ["magic", "truncate", "len12", "kraft", "tile_off", "tile_off_end",
                                  "shape", "region", "split", "split_order", "parts"])
def test_corrupt_images_rejected(what):
    b, img, info = _image()
    img = img.copy()
    off = info["region_offset"]
    expect = dg.LW_E_FORMAT
    if what == "magic":
        img[0] ^= 0xFF
    elif what == "truncate":
        img = img[: len(img) // 2]
    elif what == "len12":
        # move a symbol from length 11 to a (nonexistent) 12th length slot is not
        # representable; corrupt count[11] instead so the Kraft sum breaks
        t = img[off[dg.LW_REG_TABLE]:].view(np.uint16)
        t[11] += 1
        expect = dg.LW_E_TABLE
    elif what == "kraft":
        t = img[off[dg.LW_REG_TABLE]:].view(np.uint16)
        t[24 + 5] ^= 0x40          # a limit[] entry no longer consistent
        expect = dg.LW_E_TABLE
    elif what == "tile_off":
        to = img[off[dg.LW_REG_TILE_OFF]:].view(np.uint32)
        to[3] += 1
    elif what == "tile_off_end":
        to = img[off[dg.LW_REG_TILE_OFF]:].view(np.uint32)
        to[info["n_tiles"]] += 32
    elif what == "shape":
        img[16:24] = np.frombuffer(np.int64(100).tobytes(), np.uint8)   # rows = 100
    elif what == "region":
        hdr = img[:512].view(np.uint64)
        # the header's region offset array starts at byte 104; push the words region past the end
        assert hdr[104 // 8 + dg.LW_REG_WORDS] == off[dg.LW_REG_WORDS]
        hdr[104 // 8 + dg.LW_REG_WORDS] = len(img) + 4096
    elif what == "split":
        sp = img[off[dg.LW_REG_SPLIT]:].view(np.uint16)
        sp[5] = 0xFFFF                # a part starting past the lane's words
    elif what == "split_order":
        assert info["parts"] > 1
        sp = img[off[dg.LW_REG_SPLIT]:].view(np.uint16)
        sp[32 + 3] = sp[3]            # part 2 of lane 3 starting where part 1 does
    elif what == "parts":
        hdr = img[:512].view(np.int32)
        # the parts field follows the region offset and size arrays (bytes 104 .. 296)
        assert hdr[296 // 4] == info["parts"]
        hdr[296 // 4] = 3
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_load(img)
    assert e.value.status == expect, (what, e.value)


REGION_NAMES = ["table", "gputab", "tile_off", "words", "dm", "palette", "sm", "vb_bits", "vb_start",
                "verbatim", "split", "work"]


@pytest.mark.parametrize("kind", ["q4", "bf16"])
def test_missing_region_rejected(kind):
    """An image without a region some kernel of its kind reads is refused
    (LW_E_FORMAT, the region named) -- the same requirement table the launch
    paths check before they enqueue anything, so a kernel never reads an
    absent region through a null pointer."""
    if kind == "q4":
        codes, d, m, _ = synth.gen_q_custom(128, 1280, 71)          # five column blocks: a workspace
        b = dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m)
        needed = ["table", "gputab", "tile_off", "words", "dm", "split", "work"]
    else:
        w, _ = synth.gen_bf16_custom(128, 1280, 72, outlier_frac=0.02)
        b = dg.lw_bundle_build_bf16(w)
        needed = ["table", "gputab", "tile_off", "words", "palette", "sm", "vb_bits", "vb_start", "verbatim",
                  "split", "work"]
    info = dg.lw_bundle_get_info(b)
    assert info["n_cb"] > 4 and (kind == "q4" or info["n_verbatim"] > 0)
    base = dg.lw_bundle_image(b)
    for name in needed:
        r = REGION_NAMES.index(name)
        img = base.copy()
        hdr = img[:512].view(np.uint64)
        hdr[104 // 8 + r] = 0                      # offset
        hdr[200 // 8 + r] = 0                      # size
        with pytest.raises(dg.LwError) as e:
            dg.lw_bundle_load(img)
        assert e.value.status == dg.LW_E_FORMAT, name
        assert name in str(e.value), (name, str(e.value))


# ------------------------------------------------------------------ tile-skipping fixed-width twin

@pytest.mark.parametrize("bits,rows,cols,seed", [(2, 128, 512, 61), (4, 192, 768, 62), (8, 64, 1280, 63),
                                                 (4, 320, 2304, 64)])
def test_skip_pack_matches_oracle_bytes(bits, rows, cols, seed):
    """The product packer and the oracle write the same tile-transposed words and scales."""
    codes, d, m, _ = synth.gen_fixed(rows, cols, bits, seed)
    w, dm = dg.lw_skip_pack(codes, bits, d, m)
    ow, odm = O.skip_pack(codes, bits, d, m)
    assert np.array_equal(w, ow) and np.array_equal(dm, odm)


def test_skip_argument_rules():
    from decode_gemv_amd import lw
    codes, d, m, _ = synth.gen_fixed(64, 256, 4, 65)
    with pytest.raises(dg.LwError) as e:
        dg.lw_skip_pack(codes, 3, d, m)
    assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:
        dg.lw_skip_pack(np.full((64, 256), 4, np.uint8), 2, d, m)       # 4 does not fit in 2 bits
    assert e.value.status == dg.LW_E_ARG
    # host-side checks of lw_skip_gemv: each returns before any HIP call
    f = lw._L.lw_skip_gemv
    assert f(None, None, 4, 64, 256, None, 0, None, None, 1, None) == dg.LW_OK       # empty list
    assert f(None, None, 4, 64, 256, None, -1, None, None, 1, None) == dg.LW_E_ARG
    assert f(None, None, 3, 64, 256, None, 1, None, None, 1, None) == dg.LW_E_ARG
    assert f(None, None, 4, 65, 256, None, 1, None, None, 1, None) == dg.LW_E_SHAPE
    assert f(None, None, 4, 64, 200, None, 1, None, None, 1, None) == dg.LW_E_SHAPE
    assert f(None, None, 4, 64, 256, None, 1, None, None, 5, None) == dg.LW_E_ARG
    assert f(None, None, 4, 64, 256, None, 1, None, None, 1, None) == dg.LW_E_ARG     # null pointers


@pytest.mark.parametrize("halves", [1, 2])
@pytest.mark.parametrize("kind,law,rows,cols,seed", [
    (dg.LW_Q4_PAIR, "normal", 192, 768, 81), (dg.LW_Q4_PAIR, "uniform", 64, 512, 82),
    (dg.LW_Q4_PAIR, "const", 128, 256, 83), (dg.LW_Q6_SINGLE, "normal", 128, 1280, 84),
    (dg.LW_Q4_PAIR, "laplace", 320, 2304, 85)])
def test_rans_build_matches_oracle(kind, law, rows, cols, seed, halves):
    """The product's rANS builder writes the oracle's frequencies, offsets and
    words bit for bit, and its kernel table maps every slot to the oracle's
    symbol, frequency and slot - cum."""
    qmax, mu, sc = (15, 7.5, 1.8) if kind == dg.LW_Q4_PAIR else (63, 31.5, 5.0)
    if law == "laplace":
        sc = 1.2
    codes, _, _, _ = synth.gen_q_custom(rows, cols, seed, qmax=qmax, law=law, mu=mu, scale=sc)
    p = dg.lw_rans_build(kind, codes, halves)
    o = O.build_rans_q(O.Q4 if kind == dg.LW_Q4_PAIR else O.Q6, codes, halves)
    assert np.array_equal(p["freq"], o["f"])
    assert np.array_equal(p["tile_off"], o["tile_off"])
    assert np.array_equal(p["words"], o["words"])
    blocks = np.diff(o["tile_off"].astype(np.int64))
    assert p["max_tile_words"] == int(blocks.max())
    lut = p["lut"].reshape(2048, 2)
    slot = np.arange(2048)
    sym = np.searchsorted(o["cum"].astype(np.int64), slot, side="right") - 1
    # the search lands on the last symbol with cum <= slot, which has f > 0
    assert np.all(o["f"][sym] > 0)
    assert np.array_equal(lut[:, 0] & 0xFFF, o["f"][sym])
    assert np.array_equal(lut[:, 0] >> 24, sym)
    assert np.array_equal(lut[:, 1], slot - o["cum"][sym])
    assert not np.any(lut[:, 0] & 0x00FFF000)


def test_rans_argument_rules():
    from decode_gemv_amd import lw
    codes = np.zeros((64, 256), np.uint8)
    with pytest.raises(dg.LwError) as e:
        dg.lw_rans_build(dg.LW_BF16_EXP, codes)
    assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:
        dg.lw_rans_build(dg.LW_Q4_PAIR, np.full((64, 256), 16, np.uint8))
    assert e.value.status == dg.LW_E_ARG
    with pytest.raises(dg.LwError) as e:
        dg.lw_rans_build(dg.LW_Q4_PAIR, np.zeros((64, 200), np.uint8))
    assert e.value.status == dg.LW_E_SHAPE
    # words_cap below the size the sizing pass reports
    f16, lut, to = np.zeros(256, np.uint16), np.zeros(4096, np.uint32), np.zeros(2, np.uint32)
    nw, mt = ctypes.c_int64(), ctypes.c_int32()
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    small = np.zeros(8, np.uint32)
    assert lw._L.lw_rans_build(1, 64, 256, vp(codes), 1, vp(f16), vp(lut), vp(to), vp(small), 8, ctypes.byref(nw),
                               ctypes.byref(mt)) == dg.LW_E_ARG
    assert lw._L.lw_rans_build(1, 64, 256, vp(codes), 3, vp(f16), vp(lut), vp(to), None, 0, ctypes.byref(nw),
                               ctypes.byref(mt)) == dg.LW_E_ARG                                   # halves
    # host-side checks of lw_rans_decode: each returns before any HIP call
    f = lw._L.lw_rans_decode
    assert f(3, 64, 256, 1, None, None, None, 64, None, 0, None, None) == dg.LW_E_ARG         # kind
    assert f(1, 64, 200, 1, None, None, None, 64, None, 0, None, None) == dg.LW_E_SHAPE
    assert f(1, 64, 256, 3, None, None, None, 64, None, 0, None, None) == dg.LW_E_ARG         # halves
    assert f(1, 64, 256, 1, None, None, None, 80, None, 0, None, None) == dg.LW_E_ARG         # not 64 + 32k
    assert f(1, 64, 256, 1, None, None, None, 64 + 32 * 129, None, 0, None, None) == dg.LW_E_ARG
    assert f(1, 64, 256, 2, None, None, None, 64, None, 0, None, None) == dg.LW_E_ARG         # below 128 states
    assert f(1, 64, 256, 1, None, None, None, 64, None, 0, None, None) == dg.LW_E_ARG         # null pointers


def test_recon_argument_rules():
    """Host-side checks of the transcode and reconstructive GEMM entry points
    (each returns before any HIP call)."""
    from decode_gemv_amd import lw
    assert lw._L.lw_bf16_transcode(None, 0, None, 0, None, 0, None) == dg.LW_E_ARG
    assert lw._L.lw_recon_gemm(None, 0, None, 0, None, 0, None, None, 1, -1, None, 0, None) == dg.LW_E_ARG
    assert lw._L.lw_bundle_attach_palette(None, None, 0, None) == dg.LW_E_ARG
    assert lw._L.lw_pipeline_scratch_bytes(None, dg.LW_PIPE_PALETTE) == 0
    assert dg.LW_PIPE_COUNT == 5 and dg.LW_RECON_VARIANTS == 5
