"""Python binding of liblw (include/lw.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Host arrays are
numpy; device memory and streams come from PyTorch (a uint8 CUDA tensor for a
bundle image, fp16/bf16/fp32 CUDA tensors for x and y, the current stream).
All compute runs in the HIP kernels of liblw; if the library is missing the
import of this module fails.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblw.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "lw.h")

LW_OK, LW_E_ARG, LW_E_SHAPE, LW_E_TABLE, LW_E_FORMAT, LW_E_NOMEM, LW_E_DEVICE, LW_E_UNSUPPORTED = range(8)
LW_Q4_PAIR, LW_Q6_SINGLE, LW_BF16_EXP = 1, 2, 3
LW_PIPE_FUSED, LW_PIPE_FULL_DECODE, LW_PIPE_EXPONENT, LW_PIPE_PALETTE, LW_PIPE_DIRECT_PALETTE, LW_PIPE_COUNT = range(6)
LW_FORM_PALETTE, LW_FORM_EXPONENT = 0, 1
LW_CODE_HUFFMAN, LW_CODE_COMPACT, LW_CODE_LENS = 0, 1, 2
LW_RECON_VARIANTS = 5
(LW_REG_TABLE, LW_REG_GPUTAB, LW_REG_TILE_OFF, LW_REG_WORDS, LW_REG_DM, LW_REG_PALETTE, LW_REG_SM,
 LW_REG_VB_BITS, LW_REG_VB_START, LW_REG_VERBATIM, LW_REG_SPLIT, LW_REG_WORK, LW_REG_COUNT) = range(13)


class LwError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"lw status {status}: {msg}")
        self.status = status


class lw_bundle_info(C.Structure):
    _fields_ = [("kind", C.c_int32), ("bits", C.c_int32), ("rows", C.c_int64), ("cols", C.c_int64),
                ("n_tiles", C.c_int64), ("n_rb", C.c_int32), ("n_cb", C.c_int32),
                ("symbols_per_lane", C.c_int32), ("n_symbols", C.c_int32), ("min_len", C.c_int32),
                ("max_len", C.c_int32), ("max_words", C.c_int32), ("n_palette", C.c_int32),
                ("n_verbatim", C.c_int64), ("count_per_len", C.c_uint16 * 12),
                ("region_offset", C.c_uint64 * LW_REG_COUNT), ("region_bytes", C.c_uint64 * LW_REG_COUNT),
                ("image_bytes", C.c_uint64), ("coded_bytes", C.c_uint64), ("twin_bytes", C.c_uint64),
                ("code", C.c_int32), ("parts", C.c_int32)]


class lw_build_opts(C.Structure):
    _fields_ = [("code", C.c_int32), ("parts", C.c_int32), ("lens", C.c_void_p)]


def _load():
    # Device memory and streams come from PyTorch, so liblw must run on the
    # same HIP runtime instance as torch: importing torch first maps torch's
    # libamdhip64, which then satisfies liblw's dependency by its soname.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m decode_gemv_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, i64, i32, st = C.c_void_p, C.c_int64, C.c_int, C.c_int
    sig = {
        "lw_bundle_build_q": (st, [i32, i64, i64, P, P, P, C.POINTER(P)]),
        "lw_bundle_build_q_compact": (st, [i32, i64, i64, P, P, P, C.POINTER(P)]),
        "lw_bundle_build_q_lens": (st, [i32, i64, i64, P, P, P, P, C.POINTER(P)]),
        "lw_bundle_build_q_opts": (st, [i32, i64, i64, P, P, P, C.POINTER(lw_build_opts), C.POINTER(P)]),
        "lw_bundle_build_bf16_opts": (st, [i64, i64, P, C.POINTER(lw_build_opts), C.POINTER(P)]),
        "lw_bundle_build_bf16": (st, [i64, i64, P, C.POINTER(P)]),
        "lw_bundle_build_bf16_compact": (st, [i64, i64, P, C.POINTER(P)]),
        "lw_bundle_load": (st, [P, C.c_size_t, C.POINTER(P)]),
        "lw_bundle_validate": (st, [P]),
        "lw_bundle_get_info": (st, [P, C.POINTER(lw_bundle_info)]),
        "lw_bundle_image": (st, [P, C.POINTER(P), C.POINTER(C.c_size_t)]),
        "lw_bundle_region": (st, [P, i32, C.POINTER(P), C.POINTER(C.c_size_t)]),
        "lw_bundle_free": (None, [P]),
        "lw_twin_build": (st, [P, i32, i64, i64, P, P, P, P]),
        "lw_bundle_upload": (st, [P, P, C.c_size_t, P, C.POINTER(P)]),
        "lw_dev_bundle_free": (None, [P]),
        "lw_gemv": (st, [P, P, P, i32, P]),
        "lw_gemv_noalloc": (st, [P, P, P, i32, P]),
        "lw_decode_only": (st, [P, P, C.c_size_t, P, P]),
        "lw_twin_gemv": (st, [P, P, i32, i64, i64, P, P, i32, P]),
        "lw_swiglu": (st, [P, P, P, i64, P]),
        "lw_skip_pack": (st, [P, i32, i64, i64, P, P, P, P]),
        "lw_skip_gemv": (st, [P, P, i32, i64, i64, P, i64, P, P, i32, P]),
        "lw_read_probe": (st, [P, C.c_size_t, P, P]),
        "lw_bf16_transcode": (st, [P, i32, P, C.c_size_t, P, C.c_size_t, P]),
        "lw_recon_gemm": (st, [P, i32, P, C.c_size_t, P, C.c_size_t, P, P, i32, i32, P, C.c_size_t, P]),
        "lw_bundle_attach_palette": (st, [P, P, C.c_size_t, P]),
        "lw_pipeline_scratch_bytes": (C.c_size_t, [P, i32]),
        "lw_rans_build": (st, [i32, i64, i64, P, i32, P, P, P, P, i64, C.POINTER(C.c_int64), C.POINTER(C.c_int32)]),
        "lw_rans_decode": (st, [i32, i64, i64, i32, P, P, P, C.c_int32, P, C.c_size_t, P, P]),
        "lw_gemm_full_decode": (st, [P, P, C.c_size_t, P, P, i32, P]),
        "lw_pipeline_set": (st, [P, i32, i32, i32]),
        "lw_pipeline_get": (st, [P, i32, C.POINTER(C.c_int)]),
        "lw_gemm": (st, [P, P, P, i32, P, C.c_size_t, P]),
        "lw_autotune": (st, [P, P, i32, P, C.c_size_t, P, P, i32, P, P]),
        "lw_status_str": (C.c_char_p, [st]),
        "lw_last_error": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


_L = _load()


def lib():
    return _L


def header_functions() -> list[str]:
    """Names of the functions include/lw.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lw_[a-z0-9_]+)\s*\(", txt)))


def _check(status: int):
    if status != LW_OK:
        raise LwError(status, (_L.lw_last_error() or b"").decode())


def _np(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- host bundles

class Bundle:
    """Owner of a host lw_bundle pointer."""

    def __init__(self, ptr: int):
        self.ptr = C.c_void_p(ptr)
        self._free = _L.lw_bundle_free      # held here: module globals may be gone at interpreter exit

    def __del__(self):
        if getattr(self, "ptr", None) and self.ptr.value:
            self._free(self.ptr)
            self.ptr = None


def lw_bundle_build_q(kind: int, codes: np.ndarray, d: np.ndarray, m: np.ndarray) -> Bundle:
    rows, cols = codes.shape
    codes, pc = _np(codes, np.uint8)
    d, pd = _np(d, np.uint16)
    m, pm = _np(m, np.uint16)
    out = C.c_void_p()
    _check(_L.lw_bundle_build_q(kind, rows, cols, pc, pd, pm, C.byref(out)))
    return Bundle(out.value)


def lw_bundle_build_q_compact(kind: int, codes: np.ndarray, d: np.ndarray, m: np.ndarray) -> Bundle:
    rows, cols = codes.shape
    codes, pc = _np(codes, np.uint8)
    d, pd = _np(d, np.uint16)
    m, pm = _np(m, np.uint16)
    out = C.c_void_p()
    _check(_L.lw_bundle_build_q_compact(kind, rows, cols, pc, pd, pm, C.byref(out)))
    return Bundle(out.value)


def _lens_u8(kind: int, lens):
    n = 256 if kind == LW_Q4_PAIR else 64
    lens = np.asarray(lens)
    # the C side takes one byte per length: refuse what a cast would wrap or truncate
    if lens.dtype.kind not in "iu":
        raise ValueError("lens must be an integer array")
    if lens.size != n:
        raise ValueError(f"lens must hold {n} lengths")
    if lens.size and (lens.min() < 0 or lens.max() > 11):
        raise ValueError("code lengths must lie in 0..11")
    return _np(lens, np.uint8)


def lw_bundle_build_q_lens(kind: int, codes: np.ndarray, d: np.ndarray, m: np.ndarray, lens: np.ndarray) -> Bundle:
    rows, cols = codes.shape
    codes, pc = _np(codes, np.uint8)
    d, pd = _np(d, np.uint16)
    m, pm = _np(m, np.uint16)
    lens, pl = _lens_u8(kind, lens)
    out = C.c_void_p()
    _check(_L.lw_bundle_build_q_lens(kind, rows, cols, pc, pd, pm, pl, C.byref(out)))
    return Bundle(out.value)


def lw_bundle_build_q_opts(kind: int, codes: np.ndarray, d: np.ndarray, m: np.ndarray,
                           code: int = LW_CODE_HUFFMAN, parts: int = 0, lens=None) -> Bundle:
    rows, cols = codes.shape
    codes, pc = _np(codes, np.uint8)
    d, pd = _np(d, np.uint16)
    m, pm = _np(m, np.uint16)
    opts = lw_build_opts(code=code, parts=parts, lens=None)
    if lens is not None:
        lens, pl = _lens_u8(kind, lens)
        opts.lens = pl
    out = C.c_void_p()
    _check(_L.lw_bundle_build_q_opts(kind, rows, cols, pc, pd, pm, C.byref(opts), C.byref(out)))
    return Bundle(out.value)


def lw_bundle_build_bf16_opts(w: np.ndarray, code: int = LW_CODE_HUFFMAN, parts: int = 0) -> Bundle:
    rows, cols = w.shape
    w, pw = _np(w, np.uint16)
    opts = lw_build_opts(code=code, parts=parts, lens=None)
    out = C.c_void_p()
    _check(_L.lw_bundle_build_bf16_opts(rows, cols, pw, C.byref(opts), C.byref(out)))
    return Bundle(out.value)


def lw_bundle_build_bf16(w: np.ndarray) -> Bundle:
    rows, cols = w.shape
    w, pw = _np(w, np.uint16)
    out = C.c_void_p()
    _check(_L.lw_bundle_build_bf16(rows, cols, pw, C.byref(out)))
    return Bundle(out.value)


def lw_bundle_build_bf16_compact(w: np.ndarray) -> Bundle:
    rows, cols = w.shape
    w, pw = _np(w, np.uint16)
    out = C.c_void_p()
    _check(_L.lw_bundle_build_bf16_compact(rows, cols, pw, C.byref(out)))
    return Bundle(out.value)


def lw_bundle_load(image: np.ndarray) -> Bundle:
    image, p = _np(image, np.uint8)
    out = C.c_void_p()
    _check(_L.lw_bundle_load(p, image.nbytes, C.byref(out)))
    return Bundle(out.value)


def lw_bundle_validate(b: Bundle) -> None:
    _check(_L.lw_bundle_validate(b.ptr))


def lw_bundle_get_info(b: Bundle) -> dict:
    info = lw_bundle_info()
    _check(_L.lw_bundle_get_info(b.ptr, C.byref(info)))
    d = {k: getattr(info, k) for k, _ in lw_bundle_info._fields_}
    for k in ("count_per_len", "region_offset", "region_bytes"):
        d[k] = list(d[k])
    return d


def lw_bundle_image(b: Bundle) -> np.ndarray:
    p, n = C.c_void_p(), C.c_size_t()
    _check(_L.lw_bundle_image(b.ptr, C.byref(p), C.byref(n)))
    return np.ctypeslib.as_array((C.c_uint8 * n.value).from_address(p.value)).copy()


def lw_bundle_region(b: Bundle, region: int, dtype=np.uint8) -> np.ndarray:
    p, n = C.c_void_p(), C.c_size_t()
    _check(_L.lw_bundle_region(b.ptr, region, C.byref(p), C.byref(n)))
    if not n.value:
        return np.zeros(0, dtype=dtype)
    raw = np.ctypeslib.as_array((C.c_uint8 * n.value).from_address(p.value)).copy()
    return raw.view(dtype)


def lw_twin_build(codes: np.ndarray, bits: int, d: np.ndarray, m: np.ndarray):
    rows, cols = codes.shape
    codes, pc = _np(codes, np.uint8)
    d, pd = _np(d, np.uint16)
    m, pm = _np(m, np.uint16)
    twin = np.zeros((rows, cols // 2), np.uint8)
    dm = np.zeros((rows, cols // 256), np.uint32)
    _check(_L.lw_twin_build(pc, bits, rows, cols, pd, pm, twin.ctypes.data_as(C.c_void_p),
                            dm.ctypes.data_as(C.c_void_p)))
    return twin, dm


def lw_skip_pack(codes: np.ndarray, bits: int, d: np.ndarray, m: np.ndarray):
    """Tile-transposed words [(rows/64) * WPR * 64] and scales [(rows/64) * (cols/256) * 64]."""
    rows, cols = codes.shape
    codes, pc = _np(codes, np.uint8)
    d, pd = _np(d, np.uint16)
    m, pm = _np(m, np.uint16)
    words = np.zeros(rows * cols * bits // 32, np.uint32)
    dm = np.zeros(rows * (cols // 256), np.uint32)
    _check(_L.lw_skip_pack(pc, bits, rows, cols, pd, pm, words.ctypes.data_as(C.c_void_p),
                           dm.ctypes.data_as(C.c_void_p)))
    return words, dm


def lw_rans_build(kind: int, codes: np.ndarray, halves: int = 1) -> dict:
    """rANS twin (one stream per tile row, or two with halves=2): dict(freq, lut, tile_off, words,
    max_tile_words, halves)."""
    rows, cols = codes.shape
    codes, pc = _np(codes, np.uint8)
    n_alpha = 256 if kind == LW_Q4_PAIR else 64
    freq = np.zeros(n_alpha, np.uint16)
    lut = np.zeros(4096, np.uint32)
    tile_off = np.zeros((rows // 64) * (cols // 256) + 1, np.uint32)
    nw, mt = C.c_int64(), C.c_int32()
    vp = lambda a: a.ctypes.data_as(C.c_void_p)
    _check(_L.lw_rans_build(kind, rows, cols, pc, halves, vp(freq), vp(lut), vp(tile_off), None, 0, C.byref(nw),
                            C.byref(mt)))
    words = np.zeros(max(nw.value, 4), np.uint32)
    _check(_L.lw_rans_build(kind, rows, cols, pc, halves, vp(freq), vp(lut), vp(tile_off), vp(words), words.size,
                            C.byref(nw), C.byref(mt)))
    return dict(kind=kind, rows=rows, cols=cols, freq=freq, lut=lut, tile_off=tile_off, words=words[:nw.value],
                max_tile_words=mt.value, halves=halves)


def lw_status_str(s: int) -> str:
    return _L.lw_status_str(s).decode()


def lw_last_error() -> str:
    return (_L.lw_last_error() or b"").decode()


# ---------------------------------------------------------------- device side

def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dptr(t, what):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise LwError(LW_E_ARG, f"{what} must be a contiguous device tensor")
    return C.c_void_p(t.data_ptr())


class DevBundle:
    """Host-side descriptor of an uploaded bundle; keeps its buffer alive."""

    def __init__(self, ptr: int, buf, info: dict):
        self.ptr = C.c_void_p(ptr)
        self.buf = buf
        self.info = info
        self._free = _L.lw_dev_bundle_free  # held here: module globals may be gone at interpreter exit

    def __del__(self):
        if getattr(self, "ptr", None) and self.ptr.value:
            self._free(self.ptr)
            self.ptr = None


def lw_bundle_upload(b: Bundle, dev_buf, stream=None) -> DevBundle:
    out = C.c_void_p()
    _check(_L.lw_bundle_upload(b.ptr, _dptr(dev_buf, "dev_buf"), dev_buf.numel() * dev_buf.element_size(),
                               _stream(stream), C.byref(out)))
    return DevBundle(out.value, dev_buf, lw_bundle_get_info(b))


def lw_gemv(db: DevBundle, x, y, batch: int, stream=None) -> None:
    _check(_L.lw_gemv(db.ptr, _dptr(x, "x"), _dptr(y, "y"), batch, _stream(stream)))


def lw_gemv_noalloc(db: DevBundle, x, y, batch: int, stream=None) -> None:
    _check(_L.lw_gemv_noalloc(db.ptr, _dptr(x, "x"), _dptr(y, "y"), batch, _stream(stream)))


def lw_decode_only(db: DevBundle, out, lane_bits=None, stream=None) -> None:
    lb = _dptr(lane_bits, "lane_bits") if lane_bits is not None else None
    _check(_L.lw_decode_only(db.ptr, _dptr(out, "out"), out.numel() * out.element_size(), lb, _stream(stream)))


def lw_twin_gemv(twin, dm, bits: int, rows: int, cols: int, x, y, batch: int, stream=None) -> None:
    _check(_L.lw_twin_gemv(_dptr(twin, "twin"), _dptr(dm, "dm"), bits, rows, cols, _dptr(x, "x"), _dptr(y, "y"),
                           batch, _stream(stream)))


def lw_skip_gemv(words, dm, bits: int, rows: int, cols: int, tiles, x, y, batch: int, stream=None) -> None:
    """y rows of the listed tiles (device int32 tensor) = W x; other rows untouched."""
    n = tiles.numel()
    tp = _dptr(tiles, "tiles") if n else None
    wp = _dptr(words, "words") if n else None
    dp = _dptr(dm, "dm") if n else None
    xp = _dptr(x, "x") if n else None
    yp = _dptr(y, "y") if n else None
    _check(_L.lw_skip_gemv(wp, dp, bits, rows, cols, tp, n, xp, yp, batch, _stream(stream)))


def lw_rans_decode(kind: int, rows: int, cols: int, lut, tile_off, words, max_tile_words: int, out,
                   final_state=None, halves: int = 1, stream=None) -> None:
    """Decode the rANS twin (device tensors) into out (device uint8 tensor, the lw_decode_only layout)."""
    fp = _dptr(final_state, "final_state") if final_state is not None else None
    _check(_L.lw_rans_decode(kind, rows, cols, halves, _dptr(lut, "lut"), _dptr(tile_off, "tile_off"),
                             _dptr(words, "words"), max_tile_words, _dptr(out, "out"), out.numel() * out.element_size(),
                             fp, _stream(stream)))


def _wbuf(wbuf):
    return (_dptr(wbuf, "wbuf"), wbuf.numel() * wbuf.element_size()) if wbuf is not None else (None, 0)


def lw_gemm_full_decode(db: DevBundle, wbuf, x, y, batch: int, stream=None) -> None:
    wp, wn = _wbuf(wbuf)
    _check(_L.lw_gemm_full_decode(db.ptr, wp, wn, _dptr(x, "x"), _dptr(y, "y"), batch, _stream(stream)))


def lw_pipeline_set(db: DevBundle, batch_lo: int, batch_hi: int, pipeline: int) -> None:
    _check(_L.lw_pipeline_set(db.ptr, batch_lo, batch_hi, pipeline))


def lw_pipeline_get(db: DevBundle, batch: int) -> int:
    p = C.c_int()
    _check(_L.lw_pipeline_get(db.ptr, batch, C.byref(p)))
    return p.value


def lw_gemm(db: DevBundle, x, y, batch: int, wbuf=None, stream=None) -> None:
    wp, wn = _wbuf(wbuf)
    _check(_L.lw_gemm(db.ptr, _dptr(x, "x"), _dptr(y, "y"), batch, wp, wn, _stream(stream)))


def lw_bf16_transcode(db: DevBundle, form: int, out, vrank, stream=None) -> None:
    """Transcode the coded exponents into the palette or exponent form (device tensors)."""
    _check(_L.lw_bf16_transcode(db.ptr, form, _dptr(out, "out"), out.numel() * out.element_size(),
                                _dptr(vrank, "vrank"), vrank.numel() * vrank.element_size(), _stream(stream)))


def lw_recon_gemm(db: DevBundle, form: int, src, vrank, x, y, batch: int, variant: int = -1, work=None,
                  stream=None) -> None:
    wp, wn = _wbuf(work)
    _check(_L.lw_recon_gemm(db.ptr, form, _dptr(src, "src"), src.numel() * src.element_size(), _dptr(vrank, "vrank"),
                            vrank.numel() * vrank.element_size(), _dptr(x, "x"), _dptr(y, "y"), batch, variant, wp, wn,
                            _stream(stream)))


def lw_bundle_attach_palette(db: DevBundle, buf, stream=None) -> None:
    """Transcode into buf once and keep it with the bundle (the buffer is held by db from here on)."""
    _check(_L.lw_bundle_attach_palette(db.ptr, _dptr(buf, "buf"), buf.numel() * buf.element_size(), _stream(stream)))
    db.palette_buf = buf


def lw_pipeline_scratch_bytes(db: DevBundle, pipeline: int) -> int:
    return int(_L.lw_pipeline_scratch_bytes(db.ptr, pipeline))


def lw_autotune(db: DevBundle, batches, x, y, wbuf=None, reps: int = 10, stream=None) -> np.ndarray:
    """Time the pipelines at each batch, set the bundle's table; returns us [n][LW_PIPE_COUNT] (-1: n/a)."""
    b = np.ascontiguousarray(batches, dtype=np.int32)
    us = np.zeros((b.size, LW_PIPE_COUNT), dtype=np.float32)
    wp, wn = _wbuf(wbuf)
    _check(_L.lw_autotune(db.ptr, b.ctypes.data_as(C.c_void_p), b.size, wp, wn, _dptr(x, "x"), _dptr(y, "y"), reps,
                          _stream(stream), us.ctypes.data_as(C.c_void_p)))
    return us


def lw_read_probe(src, sink, stream=None) -> None:
    """Read every byte of the device tensor src once (measurement only)."""
    _check(_L.lw_read_probe(_dptr(src, "src"), src.numel() * src.element_size(), _dptr(sink, "sink"),
                            _stream(stream)))


def lw_swiglu(gate, up, h, stream=None) -> None:
    """h = fp16(silu(gate) * up) elementwise; gate, up fp32 and h fp16 (int16 bits) device tensors of equal size."""
    n = gate.numel()
    if up.numel() != n or h.numel() != n:
        raise LwError(LW_E_ARG, "gate, up and h must have the same number of elements")
    _check(_L.lw_swiglu(_dptr(gate, "gate"), _dptr(up, "up"), _dptr(h, "h"), n, _stream(stream)))


# ---------------------------------------------------------------- conveniences

def upload(b: Bundle, device="cuda"):
    """Allocate a device buffer of the image size with torch and upload into it."""
    import torch
    info = lw_bundle_get_info(b)
    buf = torch.empty(int(info["image_bytes"]), dtype=torch.uint8, device=device)
    return lw_bundle_upload(b, buf)
