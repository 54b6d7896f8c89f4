// runtime.hip -- device side of the liblw C ABI: upload of a bundle image
// into caller-owned device memory, and the enqueue-only entry points that
// pick and launch the gfx950 kernels.  The library never allocates device
// memory; PyTorch (or any caller) owns buffers and streams.
#include <cstring>
#include <algorithm>
#include <map>
#include <memory>
#include <mutex>
#include <string>

#include <rocblas/rocblas.h>

#include "lane_decode.hpp"

lw_status lw_fail(lw_status s, const std::string &msg);   // bundle.cpp

// Pipeline of each batch bucket: bucket k holds batches (2^(k-1), 2^k]
// (bucket 0: batch 1), up to LW_GEMM_BATCH_MAX.
#define LW_NBUCKET 17

struct lw_dev_bundle {
    lw_image_header h;
    lw_table table;
    lw_gputab tab;
    uint8_t *base;
    int8_t pipe[LW_NBUCKET];
    int8_t variant[LW_NBUCKET];      // reconstructive GEMM variant of each bucket (-1: by batch)
    const uint32_t *pal_src;         // resident palette form (lw_bundle_attach_palette), or null
    const int32_t *pal_vrank;
    void *pal_part;                  // partial sums of the column split, in the attached buffer
    uint8_t palette[16];             // bf16: the exponent palette (host copy, for kernel arguments)
};

static lw_status hip_fail(hipError_t e, const char *what)
{
    return lw_fail(LW_E_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

template <class T>
static T *dev_region(const lw_dev_bundle *db, int r)
{
    return db->h.bytes[r] ? reinterpret_cast<T *>(db->base + db->h.off[r]) : nullptr;
}

extern "C" lw_status lw_bundle_image(const lw_bundle *b, const void **image, size_t *bytes);
extern "C" lw_status lw_bundle_validate(const lw_bundle *b);

extern "C" lw_status lw_bundle_upload(const lw_bundle *b, void *dev_buf, size_t dev_bytes, void *stream,
                                      lw_dev_bundle **out)
{
    if (!out) return lw_fail(LW_E_ARG, "out is null");
    *out = nullptr;
    if (!b || !dev_buf) return lw_fail(LW_E_ARG, "null bundle or device buffer");
    lw_status st = lw_bundle_validate(b);
    if (st) return st;
    const void *img = nullptr;
    size_t bytes = 0;
    lw_bundle_image(b, &img, &bytes);
    if (dev_bytes < bytes) return lw_fail(LW_E_ARG, "device buffer smaller than the bundle image");
    if (reinterpret_cast<uintptr_t>(dev_buf) % LW_ALIGN) return lw_fail(LW_E_ARG, "device buffer not 256-byte aligned");
    hipError_t e = hipMemcpyAsync(dev_buf, img, bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    std::unique_ptr<lw_dev_bundle> db(new lw_dev_bundle);
    std::memcpy(&db->h, img, sizeof(db->h));
    std::memcpy(&db->tab, static_cast<const uint8_t *>(img) + db->h.off[LW_REG_GPUTAB], sizeof(db->tab));
    std::memcpy(&db->table, static_cast<const uint8_t *>(img) + db->h.off[LW_REG_TABLE], sizeof(db->table));
    db->base = static_cast<uint8_t *>(dev_buf);
    for (int k = 0; k < LW_NBUCKET; k++) {    // default: the fused kernels where they exist
        db->pipe[k] = (k <= 4 || db->h.kind != LW_BF16_EXP) ? LW_PIPE_FUSED : LW_PIPE_FULL_DECODE;
        db->variant[k] = -1;
    }
    db->pal_src = nullptr;
    db->pal_vrank = nullptr;
    db->pal_part = nullptr;
    std::memset(db->palette, 0, sizeof(db->palette));
    if (db->h.bytes[LW_REG_PALETTE] >= 16)
        std::memcpy(db->palette, static_cast<const uint8_t *>(img) + db->h.off[LW_REG_PALETTE], 16);
    *out = db.release();
    return LW_OK;
}

extern "C" void lw_dev_bundle_free(lw_dev_bundle *db) { delete db; }

static KArgs make_args(const lw_dev_bundle *db)
{
    KArgs a;
    std::memset(&a, 0, sizeof(a));
    a.words = dev_region<uint32_t>(db, LW_REG_WORDS);
    a.tile_off = dev_region<uint32_t>(db, LW_REG_TILE_OFF);
    a.split = dev_region<uint16_t>(db, LW_REG_SPLIT);
    a.dm = dev_region<uint32_t>(db, LW_REG_DM);
    a.tab = dev_region<lw_gputab>(db, LW_REG_GPUTAB);
    a.sm = dev_region<uint32_t>(db, LW_REG_SM);
    a.vb_bits = dev_region<uint32_t>(db, LW_REG_VB_BITS);
    a.vb_start = dev_region<uint32_t>(db, LW_REG_VB_START);
    a.verbatim = dev_region<uint16_t>(db, LW_REG_VERBATIM);
    a.part = dev_region<float>(db, LW_REG_WORK);
    a.rows = db->h.rows;
    a.cols = db->h.cols;
    a.n_rb = db->h.n_rb;
    a.n_cb = db->h.n_cb;
    a.groups = db->h.work_groups;
    a.max_words = db->h.max_words;
    a.parts = db->h.parts;
    a.min_len = db->h.min_len;
    a.max_len = db->h.max_len;
    return a;
}

SadPlan lw_apply_plan(const lw_plan &p, KArgs &a)
{
    a.sad_k = p.sad_k;
    for (int j = 0; j < 2; j++) {
        a.c8[j] = p.c8[j];
        a.c8m1[j] = p.c8m1[j];
        a.xsel[j] = p.xsel[j];
        a.xk[j] = p.xk[j];
    }
    a.c16 = p.c16;
    a.c16m1 = p.c16m1;
    a.lut_lo = p.lut_lo;
    a.lut_hi = p.lut_hi;
    for (int r = 0; r < 4; r++) a.cbase[r] = p.cbase[r];
    a.ncmp = p.ncmp;
    SadPlan sp;
    sp.plan = p.plan;
    return sp;
}

static SadPlan plan_of(const lw_dev_bundle *db, KArgs &a)
{
    return lw_apply_plan(db->tab.plan, a);
}

static lw_status gemv_check(const lw_dev_bundle *db, const void *x, float *y, int batch)
{
    if (!db || !x || !y) return lw_fail(LW_E_ARG, "null argument");
    if (batch < 1 || batch > LW_BATCH_MAX) return lw_fail(LW_E_ARG, "batch must be in 1..16");
    if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 16)
        return lw_fail(LW_E_ARG, "x and y must be 16-byte aligned");
    return LW_OK;
}

// Refuse a launch whose kernels would read a region the bundle does not
// hold (an absent region has a null device pointer).
static lw_status require_regions(const lw_dev_bundle *db, int op, const char *what, uint32_t supplied = 0)
{
    const uint32_t need = lw_regions_needed(db->h, op) & ~supplied;
    for (int r = 0; r < LW_REG_COUNT; r++)
        if ((need >> r & 1u) && !db->h.bytes[r])
            return lw_fail(LW_E_FORMAT, std::string(what) + " reads region " + lw_region_name(r) +
                                            ", which this bundle does not hold");
    return LW_OK;
}

// Launch the GEMV kernel of a bundle's kind and the batch; a.part names the
// split-column reduction's pair slots.
static lw_status gemv_launch(const lw_dev_bundle *db, KArgs &a, const void *x, float *y, int batch, hipStream_t s)
{
    a.x = static_cast<const uint16_t *>(x);
    a.y = y;
    a.batch = batch;
    hipError_t e;
    a.pal0 = db->h.kind == LW_BF16_EXP ? db->tab.payload[0] >> 7 : 0u;
    if (batch >= 8)                        // a real dense contraction: matrix cores
        e = lw_launch_gemv_mfma(a, db->h.kind, plan_of(db, a), batch, s);
    else if (db->h.kind == LW_BF16_EXP)
        e = lw_launch_gemv_bf16(a, plan_of(db, a), batch, s);
    else
        e = lw_launch_gemv_q(a, db->h.kind, plan_of(db, a), batch, s);
    if (e == hipErrorNotSupported) return lw_fail(LW_E_UNSUPPORTED, "no kernel for this kind and batch");
    if (e != hipSuccess) return hip_fail(e, "gemv launch");
    return LW_OK;
}

extern "C" lw_status lw_gemv(const lw_dev_bundle *db, const void *x, float *y, int batch, void *stream)
{
    lw_status st = gemv_check(db, x, y, batch);
    if (st) return st;
    if ((st = require_regions(db, LW_OP_GEMV, "lw_gemv"))) return st;
    KArgs a = make_args(db);
    return gemv_launch(db, a, x, y, batch, (hipStream_t)stream);
}

// ------------------------------------------------ lw_gemv without a workspace
// The split-column reduction's pair slots live in a file-scope device array
// instead of the bundle's workspace region.  Each device holds its own copy
// of the array; host code uses only the address hipGetSymbolAddress returns
// for the current device (the array's name is a host-side stand-in there),
// looked up once per device.  The slots must be empty (zero) when a call
// starts: the array starts zeroed, and every call leaves each slot it used
// empty again (both members of every pair always arrive), so no clearing
// launch is needed.
#define LW_NOALLOC_SCRATCH_BYTES (16u << 20)
static __device__ __align__(256) uint8_t scratch[LW_NOALLOC_SCRATCH_BYTES];

namespace {

struct DeviceScratch {
    std::once_flag once;
    uint8_t *ptr = nullptr;
    hipError_t err = hipSuccess;
};

// The current device's scratch address (looked up on its first use there).
hipError_t device_scratch(uint8_t **out)
{
    constexpr int MAXDEV = 64;
    static DeviceScratch per_dev[MAXDEV];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
    DeviceScratch &d = per_dev[dev];
    std::call_once(d.once, [&d]() {
        void *p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        d.ptr = d.err == hipSuccess ? static_cast<uint8_t *>(p) : nullptr;
    });
    *out = d.ptr;
    return d.ptr ? d.err : (d.err != hipSuccess ? d.err : hipErrorInvalidSymbol);
}

}  // namespace

extern "C" lw_status lw_gemv_noalloc(const lw_dev_bundle *db, const void *x, float *y, int batch, void *stream)
{
    lw_status st = gemv_check(db, x, y, batch);
    if (st) return st;
    // the workspace comes from the scratch array, not from the bundle
    if ((st = require_regions(db, LW_OP_GEMV, "lw_gemv_noalloc", 1u << LW_REG_WORK))) return st;
    KArgs a = make_args(db);
    hipStream_t s = (hipStream_t)stream;
    const uint64_t need = db->h.bytes[LW_REG_WORK];   // pair slots (0: no split reduction)
    if (need > LW_NOALLOC_SCRATCH_BYTES)
        return lw_fail(LW_E_UNSUPPORTED, "the split-column reduction of this bundle needs " + std::to_string(need) +
                                             " bytes of scratch, more than the " +
                                             std::to_string(LW_NOALLOC_SCRATCH_BYTES) +
                                             " lw_gemv_noalloc holds; use lw_gemv");
    if (need) {
        uint8_t *sp = nullptr;
        hipError_t e = device_scratch(&sp);
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        a.part = reinterpret_cast<float *>(sp);
    }
    return gemv_launch(db, a, x, y, batch, s);
}

extern "C" lw_status lw_decode_only(const lw_dev_bundle *db, void *out, size_t out_bytes, uint32_t *lane_bits,
                                    void *stream)
{
    if (!db || !out) return lw_fail(LW_E_ARG, "null argument");
    const uint64_t need = db->h.kind == LW_Q4_PAIR ? (uint64_t)db->h.rows * db->h.cols / 2
                          : db->h.kind == LW_Q6_SINGLE ? (uint64_t)db->h.rows * db->h.cols
                                                       : (uint64_t)db->h.rows * db->h.cols * 2;
    if (out_bytes < need) return lw_fail(LW_E_ARG, "output buffer too small");
    if (reinterpret_cast<uintptr_t>(out) % 16) return lw_fail(LW_E_ARG, "output must be 16-byte aligned");
    lw_status st = require_regions(db, LW_OP_DECODE, "lw_decode_only");
    if (st) return st;
    KArgs a = make_args(db);
    a.out = out;
    a.lane_bits = lane_bits;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (db->h.kind == LW_BF16_EXP) {
        a.pal0 = db->tab.payload[0] >> 7;
        e = lw_launch_decode_bf16(a, plan_of(db, a), s);
    } else {
        e = lw_launch_decode_q(a, db->h.kind, plan_of(db, a), s);
    }
    if (e == hipErrorNotSupported) return lw_fail(LW_E_UNSUPPORTED, "no decode kernel for this kind");
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return LW_OK;
}

extern "C" lw_status lw_twin_gemv(const void *twin, const uint32_t *dm, int bits, int64_t rows, int64_t cols,
                                  const void *x, float *y, int batch, void *stream)
{
    if (!twin || !dm || !x || !y) return lw_fail(LW_E_ARG, "null argument");
    if (bits != 4) return lw_fail(LW_E_ARG, "twin supports 4-bit codes");
    if (rows <= 0 || cols <= 0 || cols % 256) return lw_fail(LW_E_SHAPE, "cols must be a multiple of 256");
    if (batch < 1 || batch > LW_BATCH_MAX) return lw_fail(LW_E_ARG, "batch must be in 1..16");
    if (reinterpret_cast<uintptr_t>(twin) % 16 || reinterpret_cast<uintptr_t>(x) % 16)
        return lw_fail(LW_E_ARG, "twin and x must be 16-byte aligned");
    hipError_t e = lw_launch_twin(static_cast<const uint8_t *>(twin), dm, rows, cols,
                                  static_cast<const uint16_t *>(x), y, batch, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "twin launch");
    return LW_OK;
}

extern "C" lw_status lw_swiglu(const float *gate, const float *up, uint16_t *h, int64_t n, void *stream)
{
    if (n < 0) return lw_fail(LW_E_ARG, "negative length");
    if (n == 0) return LW_OK;                  // nothing read or written: pointers may be null
    if (!gate || !up || !h) return lw_fail(LW_E_ARG, "null argument");
    hipError_t e = lw_launch_swiglu(gate, up, h, n, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "swiglu launch");
    return LW_OK;
}

extern "C" lw_status lw_skip_gemv(const uint32_t *words, const uint32_t *dm, int bits, int64_t rows, int64_t cols,
                                  const int32_t *tiles, int64_t n_list, const void *x, float *y, int batch,
                                  void *stream)
{
    if (n_list < 0) return lw_fail(LW_E_ARG, "negative list length");
    if (n_list > 0x3FFFFFFF) return lw_fail(LW_E_ARG, "list longer than the grid allows");
    if (bits != 2 && bits != 4 && bits != 8) return lw_fail(LW_E_ARG, "bits must be 2, 4 or 8");
    if (rows <= 0 || cols <= 0 || rows % 64 || cols % 256)
        return lw_fail(LW_E_SHAPE, "rows must be a multiple of 64 and cols of 256");
    if (rows / 64 > 0x7FFFFFFF) return lw_fail(LW_E_SHAPE, "too many tiles");
    if (batch < 1 || batch > 4) return lw_fail(LW_E_ARG, "batch must be in 1..4");
    if (n_list == 0) return LW_OK;             // an empty launch list moves nothing and writes nothing
    if (!words || !dm || !tiles || !x || !y) return lw_fail(LW_E_ARG, "null argument");
    if (reinterpret_cast<uintptr_t>(words) % 16 || reinterpret_cast<uintptr_t>(dm) % 16 ||
        reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 4 ||
        reinterpret_cast<uintptr_t>(tiles) % 4)
        return lw_fail(LW_E_ARG, "words, dm and x must be 16-byte aligned, y and tiles 4-byte aligned");
    hipError_t e = lw_launch_skip(words, dm, bits, rows, cols, tiles, n_list, static_cast<const uint16_t *>(x), y,
                                  batch, (hipStream_t)stream);
    if (e == hipErrorNotSupported)
        return lw_fail(LW_E_UNSUPPORTED, "staged activations (2 * cols * batch bytes) exceed the LDS");
    if (e != hipSuccess) return hip_fail(e, "skip launch");
    return LW_OK;
}

extern "C" lw_status lw_rans_decode(int kind, int64_t rows, int64_t cols, int halves, const uint32_t *lut,
                                    const uint32_t *tile_off, const uint32_t *words, int32_t max_tile_words, void *out,
                                    size_t out_bytes, uint32_t *final_state, void *stream)
{
    if (kind != LW_Q4_PAIR && kind != LW_Q6_SINGLE) return lw_fail(LW_E_ARG, "kind must be LW_Q4_PAIR or LW_Q6_SINGLE");
    if (rows <= 0 || cols <= 0 || rows % 64 || cols % 256)
        return lw_fail(LW_E_SHAPE, "rows must be a multiple of 64 and cols of 256");
    if (halves != 1 && halves != 2) return lw_fail(LW_E_ARG, "halves must be 1 or 2");
    const int spr = kind == LW_Q4_PAIR ? 128 : 256, ns = 64 * halves;
    const int64_t ncb = cols / 256, nt = (rows / 64) * ncb;
    if (ncb > 0x7FFFFFFF || nt > 0x7FFFFFFFll * 4) return lw_fail(LW_E_SHAPE, "too many tiles");
    if (max_tile_words < ns || max_tile_words > ns + ns / 2 * (spr / halves) || (max_tile_words - ns) % (ns / 2))
        return lw_fail(LW_E_ARG, "max_tile_words must be ns + (ns/2) k with k <= symbols per stream");
    if (!lut || !tile_off || !words || !out) return lw_fail(LW_E_ARG, "null argument");
    const int64_t stride = kind == LW_Q4_PAIR ? cols / 2 : cols;
    if (out_bytes < (size_t)(rows * stride)) return lw_fail(LW_E_ARG, "out_bytes too small");
    if (reinterpret_cast<uintptr_t>(lut) % 16 || reinterpret_cast<uintptr_t>(words) % 16 ||
        reinterpret_cast<uintptr_t>(out) % 16 || reinterpret_cast<uintptr_t>(tile_off) % 4 ||
        reinterpret_cast<uintptr_t>(final_state) % 4)
        return lw_fail(LW_E_ARG, "lut, words and out must be 16-byte aligned, tile_off and final_state 4-byte");
    hipError_t e = lw_launch_rans_decode(spr, halves, lut, tile_off, words, static_cast<uint8_t *>(out), final_state,
                                         nt, (int)ncb, stride, max_tile_words, (hipStream_t)stream);
    if (e == hipErrorNotSupported) return lw_fail(LW_E_UNSUPPORTED, "tile blocks exceed the LDS");
    if (e != hipSuccess) return hip_fail(e, "rANS decode launch");
    return LW_OK;
}

extern "C" lw_status lw_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream)
{
    if (!src || !sink) return lw_fail(LW_E_ARG, "null argument");
    if (bytes < 16 || bytes % 16) return lw_fail(LW_E_ARG, "bytes must be a positive multiple of 16");
    if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(sink) % 4)
        return lw_fail(LW_E_ARG, "src must be 16-byte aligned and sink 4-byte aligned");
    hipError_t e = lw_launch_read_probe(src, (int64_t)bytes, sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "read probe launch");
    return LW_OK;
}

// ------------------------------------------------------------------ pipelines
// "Unweight", section "Four approaches to using compressed weights": full
// decode reconstructs the bf16 weights into memory and hands them to a
// library GEMM; the fused path never materialises them.  Which one is faster
// depends on the batch and the matrix, so a per-bundle table, filled by
// measurement (lw_autotune), picks the pipeline of each batch bucket.

static int batch_bucket(int batch)
{
    int k = 0;
    while ((1 << k) < batch) k++;
    return k;
}

// one rocBLAS handle per thread and device (rocBLAS handles are not safe to
// share between threads; each keeps rocBLAS's own workspace)
static lw_status blas_handle(rocblas_handle *out)
{
    thread_local std::map<int, rocblas_handle> handles;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    auto it = handles.find(dev);
    if (it == handles.end()) {
        rocblas_handle h = nullptr;
        if (rocblas_create_handle(&h) != rocblas_status_success)
            return lw_fail(LW_E_DEVICE, "rocblas_create_handle failed");
        it = handles.emplace(dev, h).first;
    }
    *out = it->second;
    return LW_OK;
}

static bool valid_pipeline(const lw_dev_bundle *db, int pipeline, int batch)
{
    if (pipeline == LW_PIPE_FUSED) return batch <= LW_BATCH_MAX;
    if (pipeline == LW_PIPE_FULL_DECODE || pipeline == LW_PIPE_EXPONENT || pipeline == LW_PIPE_PALETTE)
        return db->h.kind == LW_BF16_EXP;
    if (pipeline == LW_PIPE_DIRECT_PALETTE) return db->h.kind == LW_BF16_EXP && db->pal_src;
    return false;
}

// ------------------------------------------------------------------ reconstructive GEMM
// "Unweight", "Four approaches to using compressed weights" and "How
// reconstructive matmul works": the exponent-only and palette pipelines
// transcode the coded exponents into a compact form (exponent bytes, or
// 4-bit palette indices) and a matrix-core GEMM rebuilds the bf16 weights
// on chip from that form and the bundle's sign+mantissa bytes.

static uint64_t form_bytes(const lw_dev_bundle *db, int form)
{
    return (uint64_t)db->h.rows * db->h.cols / (form == LW_FORM_PALETTE ? 2 : 1);
}

static uint64_t vrank_bytes(const lw_dev_bundle *db) { return (uint64_t)db->h.n_tiles * 256 * 4; }

static uint64_t round256(uint64_t v) { return (v + 255) & ~(uint64_t)255; }

extern "C" lw_status lw_bf16_transcode(const lw_dev_bundle *db, int form, void *out, size_t out_bytes, int32_t *vrank,
                                       size_t vrank_size, void *stream)
{
    if (!db || !out || !vrank) return lw_fail(LW_E_ARG, "null argument");
    if (db->h.kind != LW_BF16_EXP) return lw_fail(LW_E_UNSUPPORTED, "transcode is for bf16 bundles");
    if (form != LW_FORM_PALETTE && form != LW_FORM_EXPONENT) return lw_fail(LW_E_ARG, "unknown form");
    if (out_bytes < form_bytes(db, form) || vrank_size < vrank_bytes(db))
        return lw_fail(LW_E_ARG, "output buffer too small");
    if (reinterpret_cast<uintptr_t>(out) % 16 || reinterpret_cast<uintptr_t>(vrank) % 16)
        return lw_fail(LW_E_ARG, "out and vrank must be 16-byte aligned");
    lw_status st = require_regions(db, LW_OP_DECODE, "lw_bf16_transcode");
    if (st) return st;
    KArgs a = make_args(db);
    a.out = out;
    a.vrank = vrank;
    a.pal0 = db->tab.payload[0] >> 7;
    hipError_t e = lw_launch_transcode_bf16(a, plan_of(db, a), form == LW_FORM_EXPONENT, (hipStream_t)stream);
    if (e == hipErrorNotSupported) return lw_fail(LW_E_UNSUPPORTED, "no transcode kernel for this table");
    if (e != hipSuccess) return hip_fail(e, "transcode launch");
    return LW_OK;
}

// variant by batch when the caller leaves it open: the batch tile that holds
// the batch, up to 64 with the rows split, beyond with the batch split
static int recon_variant_for(int batch)
{
    return batch <= 16 ? 0 : batch <= 32 ? 1 : batch <= 64 ? 2 : batch <= 128 ? 3 : 4;
}

// batch columns of a workgroup in each variant
static int recon_tile(int variant) { return variant < 3 ? 16 << variant : 64 * (2 << (variant - 3)); }

// bytes of partial sums the pipelines keep room for: 8 splits of 64 batch columns
static uint64_t part_bytes(const lw_dev_bundle *db) { return (uint64_t)8 * 64 * db->h.rows * 4; }

extern "C" lw_status lw_recon_gemm(const lw_dev_bundle *db, int form, const void *src, size_t src_bytes,
                                   const int32_t *vrank, size_t vrank_size, const void *x, float *y, int batch,
                                   int variant, void *work, size_t work_bytes, void *stream)
{
    if (!db || !src || !vrank || !x || !y) return lw_fail(LW_E_ARG, "null argument");
    if (db->h.kind != LW_BF16_EXP) return lw_fail(LW_E_UNSUPPORTED, "reconstructive GEMM is for bf16 bundles");
    if (form != LW_FORM_PALETTE && form != LW_FORM_EXPONENT) return lw_fail(LW_E_ARG, "unknown form");
    if (src_bytes < form_bytes(db, form) || vrank_size < vrank_bytes(db))
        return lw_fail(LW_E_ARG, "form or rank buffer smaller than the bundle needs");
    if (batch < 1 || batch > LW_GEMM_BATCH_MAX) return lw_fail(LW_E_ARG, "batch must be in 1..65536");
    if (variant < -1 || variant >= LW_RECON_VARIANTS) return lw_fail(LW_E_ARG, "unknown variant");
    if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(vrank) % 4 ||
        reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 16)
        return lw_fail(LW_E_ARG, "src, x and y must be 16-byte aligned, vrank 4-byte aligned");
    if (variant < 0) variant = recon_variant_for(batch);
    // split the column blocks when the grid would leave the chip short of
    // wavefronts (about four per SIMD wanted) and the partial sums fit `work`
    const int64_t waves = db->h.n_rb * 4 * (((int64_t)batch + recon_tile(variant) - 1) / recon_tile(variant));
    int splits = (int)std::min<int64_t>({(int64_t)db->h.n_cb, 8, (4096 + waves - 1) / waves});
    if (!work || reinterpret_cast<uintptr_t>(work) % 16) splits = 1;
    while (splits > 1 && (uint64_t)splits * batch * db->h.rows * 4 > work_bytes) splits--;
    hipError_t e = lw_launch_recon(form == LW_FORM_EXPONENT, static_cast<const uint32_t *>(src),
                                   dev_region<uint32_t>(db, LW_REG_SM), vrank, dev_region<uint32_t>(db, LW_REG_VB_START),
                                   dev_region<uint16_t>(db, LW_REG_VERBATIM), db->h.n_verbatim,
                                   db->palette, static_cast<const uint16_t *>(x), y, db->h.rows, db->h.cols, batch,
                                   variant, static_cast<float *>(work), splits, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "reconstructive GEMM launch");
    return LW_OK;
}

extern "C" lw_status lw_bundle_attach_palette(lw_dev_bundle *db, void *buf, size_t bytes, void *stream)
{
    if (!db || !buf) return lw_fail(LW_E_ARG, "null argument");
    if (db->h.kind != LW_BF16_EXP) return lw_fail(LW_E_UNSUPPORTED, "the palette form is for bf16 bundles");
    const uint64_t sb = round256(form_bytes(db, LW_FORM_PALETTE));
    if (bytes < sb + round256(vrank_bytes(db)) + part_bytes(db))
        return lw_fail(LW_E_ARG, "buffer smaller than lw_pipeline_scratch_bytes(db, LW_PIPE_DIRECT_PALETTE)");
    if (reinterpret_cast<uintptr_t>(buf) % 256) return lw_fail(LW_E_ARG, "buffer must be 256-byte aligned");
    uint8_t *b = static_cast<uint8_t *>(buf);
    lw_status st = lw_bf16_transcode(db, LW_FORM_PALETTE, b, sb, reinterpret_cast<int32_t *>(b + sb),
                                     vrank_bytes(db), stream);
    if (st) return st;
    db->pal_src = reinterpret_cast<const uint32_t *>(b);
    db->pal_vrank = reinterpret_cast<const int32_t *>(b + sb);
    db->pal_part = b + sb + round256(vrank_bytes(db));
    return LW_OK;
}

extern "C" size_t lw_pipeline_scratch_bytes(const lw_dev_bundle *db, int pipeline)
{
    if (!db || db->h.kind != LW_BF16_EXP) return 0;
    switch (pipeline) {
    case LW_PIPE_FULL_DECODE: return (size_t)db->h.rows * db->h.cols * 2;
    case LW_PIPE_EXPONENT:
        return (size_t)(round256(form_bytes(db, LW_FORM_EXPONENT)) + round256(vrank_bytes(db)) + part_bytes(db));
    case LW_PIPE_PALETTE:
    case LW_PIPE_DIRECT_PALETTE:
        return (size_t)(round256(form_bytes(db, LW_FORM_PALETTE)) + round256(vrank_bytes(db)) + part_bytes(db));
    }
    return 0;
}

// transcode into the caller's scratch, then the reconstructive GEMM
static lw_status transcode_gemm(const lw_dev_bundle *db, int form, void *wbuf, size_t wbuf_bytes, const void *x,
                                float *y, int batch, int variant, void *stream)
{
    if (!wbuf) return lw_fail(LW_E_ARG, "null scratch buffer");
    const uint64_t sb = round256(form_bytes(db, form)), vb = round256(vrank_bytes(db));
    if (wbuf_bytes < sb + vb) return lw_fail(LW_E_ARG, "scratch buffer too small for the pipeline");
    if (reinterpret_cast<uintptr_t>(wbuf) % 256) return lw_fail(LW_E_ARG, "scratch buffer must be 256-byte aligned");
    uint8_t *b = static_cast<uint8_t *>(wbuf);
    int32_t *vr = reinterpret_cast<int32_t *>(b + sb);
    lw_status st = lw_bf16_transcode(db, form, b, sb, vr, vrank_bytes(db), stream);
    if (st) return st;
    return lw_recon_gemm(db, form, b, sb, vr, vrank_bytes(db), x, y, batch, variant, b + sb + vb, wbuf_bytes - sb - vb,
                         stream);
}

static lw_status run_pipeline(const lw_dev_bundle *db, int p, int variant, const void *x, float *y, int batch,
                              void *wbuf, size_t wbuf_bytes, void *stream)
{
    switch (p) {
    case LW_PIPE_FUSED:
        if (batch > LW_BATCH_MAX) return lw_fail(LW_E_UNSUPPORTED, "no pipeline for this batch");
        return lw_gemv(db, x, y, batch, stream);
    case LW_PIPE_FULL_DECODE: return lw_gemm_full_decode(db, wbuf, wbuf_bytes, x, y, batch, stream);
    case LW_PIPE_EXPONENT: return transcode_gemm(db, LW_FORM_EXPONENT, wbuf, wbuf_bytes, x, y, batch, variant, stream);
    case LW_PIPE_PALETTE: return transcode_gemm(db, LW_FORM_PALETTE, wbuf, wbuf_bytes, x, y, batch, variant, stream);
    case LW_PIPE_DIRECT_PALETTE:
        if (!db->pal_src) return lw_fail(LW_E_UNSUPPORTED, "no palette form attached");
        return lw_recon_gemm(db, LW_FORM_PALETTE, db->pal_src, form_bytes(db, LW_FORM_PALETTE), db->pal_vrank,
                             vrank_bytes(db), x, y, batch, variant, db->pal_part, (size_t)part_bytes(db), stream);
    }
    return lw_fail(LW_E_ARG, "unknown pipeline");
}

extern "C" lw_status lw_gemm_full_decode(const lw_dev_bundle *db, void *wbuf, size_t wbuf_bytes, const void *x,
                                         float *y, int batch, void *stream)
{
    if (!db || !wbuf || !x || !y) return lw_fail(LW_E_ARG, "null argument");
    if (db->h.kind != LW_BF16_EXP)
        return lw_fail(LW_E_UNSUPPORTED, "full decode is for bf16 bundles (their decoded weights are exact)");
    if (batch < 1 || batch > LW_GEMM_BATCH_MAX) return lw_fail(LW_E_ARG, "batch must be in 1..65536");
    const uint64_t need = (uint64_t)db->h.rows * db->h.cols * 2;
    if (wbuf_bytes < need) return lw_fail(LW_E_ARG, "weight buffer smaller than rows * cols * 2 bytes");
    if (reinterpret_cast<uintptr_t>(wbuf) % 16 || reinterpret_cast<uintptr_t>(x) % 16 ||
        reinterpret_cast<uintptr_t>(y) % 16)
        return lw_fail(LW_E_ARG, "wbuf, x and y must be 16-byte aligned");
    if (db->h.rows > 0x7FFFFFFF || db->h.cols > 0x7FFFFFFF) return lw_fail(LW_E_SHAPE, "matrix too large for the GEMM");
    lw_status st = lw_decode_only(db, wbuf, wbuf_bytes, nullptr, stream);
    if (st) return st;
    rocblas_handle h;
    if ((st = blas_handle(&h))) return st;
    if (rocblas_set_stream(h, (hipStream_t)stream) != rocblas_status_success)
        return lw_fail(LW_E_DEVICE, "rocblas_set_stream failed");
    // column-major view: Y^T (rows x batch) = W (rows x cols) X^T (cols x batch),
    // with W row-major = A^T of a cols x rows column-major A
    const float alpha = 1.0f, beta = 0.0f;
    const rocblas_int m = (rocblas_int)db->h.rows, n = batch, k = (rocblas_int)db->h.cols;
    rocblas_status bs = rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, m, n, k, &alpha,
                                        wbuf, rocblas_datatype_bf16_r, k, x, rocblas_datatype_bf16_r, k, &beta, y,
                                        rocblas_datatype_f32_r, m, y, rocblas_datatype_f32_r, m,
                                        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    if (bs != rocblas_status_success)
        return lw_fail(LW_E_DEVICE, std::string("rocblas_gemm_ex: ") + rocblas_status_to_string(bs));
    return LW_OK;
}

extern "C" lw_status lw_pipeline_set(lw_dev_bundle *db, int batch_lo, int batch_hi, int pipeline)
{
    if (!db) return lw_fail(LW_E_ARG, "null bundle");
    if (batch_lo < 1 || batch_hi < batch_lo || batch_hi > LW_GEMM_BATCH_MAX)
        return lw_fail(LW_E_ARG, "batch range must lie in 1..65536");
    for (int k = batch_bucket(batch_lo); k <= batch_bucket(batch_hi); k++)
        if (!valid_pipeline(db, pipeline, 1 << k))
            return lw_fail(LW_E_UNSUPPORTED, "pipeline not available for this bundle and batch");
    for (int k = batch_bucket(batch_lo); k <= batch_bucket(batch_hi); k++) {
        db->pipe[k] = (int8_t)pipeline;
        db->variant[k] = -1;
    }
    return LW_OK;
}

extern "C" lw_status lw_pipeline_get(const lw_dev_bundle *db, int batch, int *pipeline)
{
    if (!db || !pipeline) return lw_fail(LW_E_ARG, "null argument");
    if (batch < 1 || batch > LW_GEMM_BATCH_MAX) return lw_fail(LW_E_ARG, "batch must be in 1..65536");
    *pipeline = db->pipe[batch_bucket(batch)];
    return LW_OK;
}

extern "C" lw_status lw_gemm(const lw_dev_bundle *db, const void *x, float *y, int batch, void *wbuf,
                             size_t wbuf_bytes, void *stream)
{
    if (!db) return lw_fail(LW_E_ARG, "null bundle");
    if (batch < 1 || batch > LW_GEMM_BATCH_MAX) return lw_fail(LW_E_ARG, "batch must be in 1..65536");
    const int k = batch_bucket(batch);
    return run_pipeline(db, db->pipe[k], db->variant[k], x, y, batch, wbuf, wbuf_bytes, stream);
}

extern "C" lw_status lw_autotune(lw_dev_bundle *db, const int *batches, int n, void *wbuf, size_t wbuf_bytes,
                                 const void *x, float *y, int reps, void *stream, float *us_out)
{
    if (!db || !batches || n < 1 || reps < 1 || !x || !y) return lw_fail(LW_E_ARG, "bad argument");
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0, e1;
    hipError_t he = hipEventCreate(&e0);
    if (he != hipSuccess) return hip_fail(he, "hipEventCreate");
    he = hipEventCreate(&e1);
    if (he != hipSuccess) {
        (void)hipEventDestroy(e0);
        return hip_fail(he, "hipEventCreate");
    }
    lw_status st = LW_OK;
    for (int i = 0; i < n && !st; i++) {
        const int batch = batches[i];
        if (batch < 1 || batch > LW_GEMM_BATCH_MAX) {
            st = lw_fail(LW_E_ARG, "batch must be in 1..65536");
            break;
        }
        float best = -1.0f;
        int best_p = -1, best_v = -1;
        for (int p = 0; p < LW_PIPE_COUNT && !st; p++) {
            if (us_out) us_out[i * LW_PIPE_COUNT + p] = -1.0f;
            if (!valid_pipeline(db, p, batch)) continue;
            if (p != LW_PIPE_FUSED && p != LW_PIPE_DIRECT_PALETTE &&
                (!wbuf || wbuf_bytes < lw_pipeline_scratch_bytes(db, p)))
                continue;                                  // no room for this pipeline's scratch
            // the reconstructive GEMM pipelines are timed in every variant
            const bool recon = p == LW_PIPE_EXPONENT || p == LW_PIPE_PALETTE || p == LW_PIPE_DIRECT_PALETTE;
            for (int v = recon ? 0 : -1; v < (recon ? LW_RECON_VARIANTS : 0) && !st; v++) {
                auto run = [&]() { return run_pipeline(db, p, v, x, y, batch, wbuf, wbuf_bytes, stream); };
                if ((st = run())) break;                   // warm-up (and first-use set-up)
                he = hipEventRecord(e0, s);
                for (int r = 0; r < reps && !st && he == hipSuccess; r++) st = run();
                if (st) break;
                if (he == hipSuccess) he = hipEventRecord(e1, s);
                if (he == hipSuccess) he = hipEventSynchronize(e1);
                float ms = 0.f;
                if (he == hipSuccess) he = hipEventElapsedTime(&ms, e0, e1);
                if (he != hipSuccess) {
                    st = hip_fail(he, "timing");
                    break;
                }
                const float us = 1000.0f * ms / (float)reps;
                if (us_out && (us_out[i * LW_PIPE_COUNT + p] < 0 || us < us_out[i * LW_PIPE_COUNT + p]))
                    us_out[i * LW_PIPE_COUNT + p] = us;
                if (best < 0 || us < best) best = us, best_p = p, best_v = v;
            }
        }
        if (!st && best_p >= 0) {
            db->pipe[batch_bucket(batch)] = (int8_t)best_p;
            db->variant[batch_bucket(batch)] = (int8_t)best_v;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return st;
}
