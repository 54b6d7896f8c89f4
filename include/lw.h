/*
 * lw.h -- C ABI of the MI355X (gfx950) library for matrix-vector products
 * over losslessly entropy-coded LLM weights.
 *
 * The method: "LazyWeights: Decode-on-Demand Edge LLMs", section "2 . Code
 * them" (one length-limited Huffman table with 11-bit codes per matrix;
 * 64x256 tiles of 32 lanes of two rows; lanes' 32-bit words interleaved;
 * 4-bit codes coded in pairs; scales and minimums kept raw), section
 * "3 . Decode on demand" and Fig. 3 (a code's length comes from comparing the
 * next 11 stream bits with per-length bounds, its symbol from that length's
 * base position in the symbol list; each tile has its own offsets and so
 * decodes independently),
 * and the runtime paragraph under Fig. 3 (software decode fused into GEMV; a
 * decode-free fixed-width "twin").  The bf16 variant follows "Unweight:
 * Compressing LLM Weights for Faster Inference", sections "Understanding BF16
 * weight structure" and "The exponent's exploitable redundancy" (only the
 * exponent byte is Huffman coded, over the matrix's top-16 palette; a 64-weight
 * row segment with an exponent outside the palette is stored verbatim; sign and
 * mantissa stay raw).  Dequantisation w = d*q - m per 256-weight super-block is
 * the grouped-storage rule of "Software-Defined Bandwidth Expansion", IV-A.
 *
 * Conventions for every entry point:
 *  - Every function returns lw_status; nothing throws across the ABI.  On an
 *    error lw_last_error() returns a thread-local detail string.
 *  - Host pointers are plain host memory; "device" pointers are HIP device
 *    addresses on the current device (PyTorch allocates them).  The library
 *    never allocates device memory and never frees caller memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  GPU
 *    entry points only enqueue work; errors found while enqueueing are
 *    returned, faults inside kernels surface at the caller's next sync.
 *  - All multi-byte values are little-endian; fp16 and bf16 values are passed
 *    as their 16-bit patterns.
 */
#ifndef LW_H
#define LW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LW_OK = 0,
    LW_E_ARG = 1,          /* null pointer, out-of-range value, buffer too small, misalignment */
    LW_E_SHAPE = 2,        /* rows not a multiple of 64 or cols not a multiple of 256 */
    LW_E_TABLE = 3,        /* code table invalid: a length above 11 or a Kraft violation */
    LW_E_FORMAT = 4,       /* bundle image corrupt or inconsistent */
    LW_E_NOMEM = 5,        /* host allocation failed */
    LW_E_DEVICE = 6,       /* a HIP call failed */
    LW_E_UNSUPPORTED = 7   /* valid request that this build does not implement */
} lw_status;

typedef enum {
    LW_Q4_PAIR = 1,        /* 4-bit codes, coded in pairs: 256-symbol alphabet, 256 symbols per lane */
    LW_Q6_SINGLE = 2,      /* 6-bit codes, coded singly: 64-symbol alphabet, 512 symbols per lane */
    LW_BF16_EXP = 3        /* bf16 weights, exponent palette index coded singly: 16 symbols, 512 per lane */
} lw_kind;

/* How a bundle's code lengths were chosen (lw_bundle_info.code). */
typedef enum {
    LW_CODE_HUFFMAN = 0,   /* the optimal prefix code with lengths <= 11 ("2 . Code them": a
                              length-limited Huffman table with 11-bit codes), by package-merge */
    LW_CODE_COMPACT = 1,   /* opt-in: the cheapest prefix code with lengths <= 11 that uses at most
                              four lengths, the three shorter <= 8 (a smaller decoder comparison plan,
                              a few tenths of a percent to two percent more bits) */
    LW_CODE_LENS = 2       /* lengths given by the caller (lw_bundle_build_q_lens) */
} lw_code;

/* Execution pipelines of lw_gemm ("Unweight", "Four approaches to using
 * compressed weights"). */
typedef enum {
    LW_PIPE_FUSED = 0,         /* decode on chip inside the GEMV (lw_gemv); batch 1..16 */
    LW_PIPE_FULL_DECODE = 1,   /* decode the weights into memory, then a library GEMM (bf16 bundles) */
    LW_PIPE_EXPONENT = 2,      /* decode the exponent bytes only, then the reconstructive GEMM (bf16) */
    LW_PIPE_PALETTE = 3,       /* transcode to 4-bit palette indices, then the reconstructive GEMM (bf16) */
    LW_PIPE_DIRECT_PALETTE = 4,/* the reconstructive GEMM over a palette form transcoded once at load (bf16) */
    LW_PIPE_COUNT = 5
} lw_pipeline;

/* Compact forms the reconstructive GEMM rebuilds bf16 weights from. */
typedef enum {
    LW_FORM_PALETTE = 0,       /* 4-bit palette index per weight */
    LW_FORM_EXPONENT = 1       /* exponent byte per weight */
} lw_form;

/* Variants of the reconstructive GEMM: 0, 1, 2 = each wavefront of a
 * workgroup multiplies 16 of its 64 rows with 16, 32 or 64 batch columns;
 * 3, 4 = each multiplies all 64 rows (rebuilt once, shared through LDS) with
 * a quarter of 128 or 256 batch columns. */
enum { LW_RECON_VARIANTS = 5 };

typedef struct lw_bundle lw_bundle;          /* host bundle: opaque, owned by the library */
typedef struct lw_dev_bundle lw_dev_bundle;  /* host-side descriptor of an uploaded bundle */

/* Region identifiers for lw_bundle_region (the image layout of a bundle). */
typedef enum {
    LW_REG_TABLE = 0,      /* canonical table: u16 count[12], first[12], limit[12], offset[12], sym_sorted[256] */
    LW_REG_GPUTAB = 1,     /* tables derived for the kernels (not part of the coded format) */
    LW_REG_TILE_OFF = 2,   /* u32 [n_tiles+1] word offset of each tile block */
    LW_REG_WORDS = 3,      /* u32 interleaved lane words; tile t's word j of lane l at tile_off[t] + 32j + l */
    LW_REG_DM = 4,         /* u32 [n_tiles][64] = d | m << 16 (fp16 bits), Q4/Q6 only */
    LW_REG_PALETTE = 5,    /* u8 [16] exponents, index 0 the most frequent (bf16 only) */
    LW_REG_SM = 6,         /* u32 [n_tiles][4096] sign+mantissa bytes, lane-interleaved (bf16 only) */
    LW_REG_VB_BITS = 7,    /* u32 [n_tiles][8], bit 4i+s marks segment s of tile row i verbatim (bf16) */
    LW_REG_VB_START = 8,   /* u32 [n_tiles+1] verbatim segments before each tile (bf16) */
    LW_REG_VERBATIM = 9,   /* u16 [n_verbatim][64] raw bf16 segments (bf16) */
    LW_REG_SPLIT = 10,     /* u16 [n_tiles][2P-1][32], P = lw_bundle_info.parts: lane stream l of a
                              tile is 2P parts of equal symbol count, P per tile row (row 2l, then
                              2l+1), and entry [t][k-1][l] is the bit where part k >= 1 begins, so
                              any part decodes on its own ("LazyWeights", Fig. 3 caption: per-tile
                              offsets let every tile start independently; here every part) */
    LW_REG_WORK = 11,      /* device workspace of the split-column reduction (zero in the image) */
    LW_REG_COUNT = 12
} lw_region;

typedef struct {
    int32_t kind;              /* lw_kind */
    int32_t bits;              /* 4, 6 or 16 */
    int64_t rows, cols;
    int64_t n_tiles;           /* (rows/64) * (cols/256), row-band-major */
    int32_t n_rb, n_cb;        /* row bands (rows/64) and column blocks (cols/256) */
    int32_t symbols_per_lane;  /* 256 (Q4) or 512 (Q6, BF16) */
    int32_t n_symbols;         /* symbols with a code */
    int32_t min_len, max_len;  /* shortest and longest code length used */
    int32_t max_words;         /* longest lane of any tile, in 32-bit words */
    int32_t n_palette;         /* bf16: distinct exponents in the palette */
    int64_t n_verbatim;        /* bf16: verbatim 64-weight segments */
    uint16_t count_per_len[12];/* index L = 1..11 */
    uint64_t region_offset[LW_REG_COUNT]; /* byte offset of each region inside the image */
    uint64_t region_bytes[LW_REG_COUNT];  /* byte size of each region (0 if absent) */
    uint64_t image_bytes;      /* size of the device image = bytes lw_bundle_upload copies/needs */
    uint64_t coded_bytes;      /* bytes a fused GEMV must read for the weights: words + tile_off + split +
                                  table + dm (Q4/Q6) or + sm + vb_bits + vb_start + verbatim +
                                  palette (bf16); excludes x, y and the workspace */
    uint64_t twin_bytes;       /* the fixed-width equivalent: rows*cols*bits/8 + rows*cols/256*4
                                  (bf16: rows*cols*2, the dense matrix) */
    int32_t code;              /* lw_code: how the code lengths were chosen */
    int32_t parts;             /* parts per tile row with a recorded start (LW_REG_SPLIT): 1, 2, 4, 8 */
} lw_bundle_info;

/* Build options (lw_bundle_build_q_opts, lw_bundle_build_bf16_opts). */
typedef struct {
    int32_t code;              /* lw_code; LW_CODE_LENS (Q4/Q6 only) takes the lengths in lens */
    int32_t parts;             /* parts per tile row whose starts are recorded: 1, 2, 4 or 8; 0 lets the
                                  library choose the largest that keeps tiles x parts <= 4096 (four
                                  wavefronts per SIMD of a 256-CU MI355X), else 1 */
    const uint8_t *lens;       /* LW_CODE_LENS: as in lw_bundle_build_q_lens; else ignored */
} lw_build_opts;

/* ---------------------------------------------------------------- host side */

/* Build a bundle from quantised codes ("2 . Code them": one length-limited
 * Huffman table per matrix, 11-bit codes; the lengths are the optimal prefix
 * code of at most 11 bits for the matrix's symbol histogram, LW_CODE_HUFFMAN).
 *   kind  : LW_Q4_PAIR or LW_Q6_SINGLE
 *   codes : host [rows][cols] row-major, one code per byte (< 16 or < 64)
 *   d, m  : host fp16 bits [rows][cols/256]: scale and minimum of each
 *           256-weight super-block; the weight is w = d*q - m
 * The inputs are copied; no caller pointer is retained.  *out receives a
 * library-owned bundle to free with lw_bundle_free.
 * Errors: LW_E_ARG (null, bad kind, a code out of range), LW_E_SHAPE,
 * LW_E_NOMEM. */
lw_status lw_bundle_build_q(int kind, int64_t rows, int64_t cols, const uint8_t *codes,
                            const uint16_t *d, const uint16_t *m, lw_bundle **out);

/* As lw_bundle_build_q with the compact code (LW_CODE_COMPACT) instead of the
 * optimal one: an opt-in that trades a little size for a decoder with one
 * pair of limit comparisons per symbol.  The bit cost is visible in
 * lw_bundle_info.coded_bytes beside the default bundle's.
 * Errors: as lw_bundle_build_q. */
lw_status lw_bundle_build_q_compact(int kind, int64_t rows, int64_t cols, const uint8_t *codes,
                                    const uint16_t *d, const uint16_t *m, lw_bundle **out);

/* As lw_bundle_build_q, with the code lengths chosen by the caller (LW_CODE_LENS)
 * instead of the library's ("2 . Code them" fixes the 11-bit limit and one
 * table per matrix): any prefix code of at most 11 bits.
 *   lens : host u8 [256] (Q4: one per pair symbol lo | hi << 4) or [64] (Q6),
 *          the code length of each symbol; a symbol that occurs needs 1..11,
 *          an absent one may have 0.  Copied, not retained.
 * Errors: as lw_bundle_build_q, LW_E_ARG for a null lens, LW_E_TABLE for a
 * missing or too long length or lengths that violate Kraft's inequality. */
lw_status lw_bundle_build_q_lens(int kind, int64_t rows, int64_t cols, const uint8_t *codes,
                                 const uint16_t *d, const uint16_t *m, const uint8_t *lens, lw_bundle **out);

/* As lw_bundle_build_q with explicit options: the code (lw_build_opts.code,
 * lens) and the parts per tile row.  More parts let more wavefronts decode
 * one tile at once (shorter serial chains, work spread evenly over the SIMDs)
 * for 2 bytes per extra part start per lane stream.  The other builders pick
 * parts = 0.  opts is read, not retained.
 * Errors: as lw_bundle_build_q_lens, LW_E_ARG for a null opts, an unknown
 * code or parts outside 0, 1, 2, 4, 8. */
lw_status lw_bundle_build_q_opts(int kind, int64_t rows, int64_t cols, const uint8_t *codes,
                                 const uint16_t *d, const uint16_t *m, const lw_build_opts *opts,
                                 lw_bundle **out);

/* Build a bf16 exponent-coded bundle ("Unweight", exponent palette and
 * verbatim rows; the palette indices coded with the optimal prefix code of at
 * most 11 bits, LW_CODE_HUFFMAN).  w: host bf16 bits [rows][cols].  Errors as
 * above. */
lw_status lw_bundle_build_bf16(int64_t rows, int64_t cols, const uint16_t *w, lw_bundle **out);

/* As lw_bundle_build_bf16 with the compact code (LW_CODE_COMPACT). */
lw_status lw_bundle_build_bf16_compact(int64_t rows, int64_t cols, const uint16_t *w, lw_bundle **out);

/* As lw_bundle_build_bf16 with explicit options (code HUFFMAN or COMPACT,
 * parts as in lw_bundle_build_q_opts).  Errors: as lw_bundle_build_bf16,
 * LW_E_ARG for bad options, LW_E_UNSUPPORTED for LW_CODE_LENS. */
lw_status lw_bundle_build_bf16_opts(int64_t rows, int64_t cols, const uint16_t *w, const lw_build_opts *opts,
                                    lw_bundle **out);

/* Re-create a bundle from an image (as returned by lw_bundle_image); the image
 * is copied and validated.  Errors: LW_E_ARG, LW_E_FORMAT, LW_E_TABLE. */
lw_status lw_bundle_load(const void *image, size_t bytes, lw_bundle **out);

/* Check every invariant of a bundle: header, region bounds, code table (Kraft
 * sum, lengths <= 11, limits), tile offsets and the longest lane.
 * Errors: LW_E_FORMAT, LW_E_TABLE. */
lw_status lw_bundle_validate(const lw_bundle *b);

lw_status lw_bundle_get_info(const lw_bundle *b, lw_bundle_info *info);

/* Pointer to the bundle's image (valid until lw_bundle_free) and its size. */
lw_status lw_bundle_image(const lw_bundle *b, const void **image, size_t *bytes);

/* Pointer to one region of the image and its size in bytes. */
lw_status lw_bundle_region(const lw_bundle *b, int region, const void **ptr, size_t *bytes);

void lw_bundle_free(lw_bundle *b);

/* Fixed-width "twin" of a quantised matrix (the decode-free stand-in of the
 * runtime paragraph under "LazyWeights" Fig. 3; grouped packing of "Software-
 * Defined Bandwidth Expansion" IV-A):
 *   bits = 4: packed [rows][cols/2] bytes, low nibble = even column.
 * dm_out receives [rows][cols/256] u32 = d | m << 16.
 * Errors: LW_E_ARG (null, bits other than 4, code >= 16), LW_E_SHAPE. */
lw_status lw_twin_build(const uint8_t *codes, int bits, int64_t rows, int64_t cols,
                        const uint16_t *d, const uint16_t *m, uint8_t *twin_out, uint32_t *dm_out);

/* ---------------------------------------------------------------- device side */

/* Copy a bundle image into caller-owned device memory dev_buf (at least
 * info.image_bytes bytes, 256-byte aligned) on `stream`, and zero its
 * workspace.  *out receives a host-side descriptor (free with
 * lw_dev_bundle_free; dev_buf must outlive it).  The host bundle may be freed
 * once the stream has passed the copy.
 * Errors: LW_E_ARG (null, buffer too small or misaligned), LW_E_DEVICE. */
lw_status lw_bundle_upload(const lw_bundle *b, void *dev_buf, size_t dev_bytes, void *stream,
                           lw_dev_bundle **out);

void lw_dev_bundle_free(lw_dev_bundle *db);

/* y = W x for an uploaded bundle, decoding the weights on chip (fused decode +
 * dequantise + dot product; HBM moves only coded bytes).
 *   x : device [batch][cols], fp16 (Q4/Q6) or bf16 (BF16) bits, 16-byte aligned
 *   y : device [batch][rows] fp32, overwritten, 16-byte aligned
 *   1 <= batch <= 16; batch >= 8 uses the matrix-core (MFMA) kernel.
 * The split-column reduction uses the bundle's workspace: calls on one
 * uploaded bundle must not overlap in time (use one stream per bundle).
 * Results are deterministic: the column groups' sums meet pairwise in a
 * fixed tree, and each pair's sum does not depend on which arrives first (an
 * output whose sum is zero may be written as -0.0).
 * Errors: LW_E_ARG, LW_E_UNSUPPORTED, LW_E_DEVICE. */
lw_status lw_gemv(const lw_dev_bundle *db, const void *x, float *y, int batch, void *stream);

/* lw_gemv for callers that cannot allocate device memory or reserve a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same kernels and results as lw_gemv, with the
 * split-column reduction's pair slots taken from a scratch array the library
 * holds per device (16 MiB, zero at load, held until the process ends)
 * instead of the bundle's workspace region.  Nothing is allocated and nothing
 * is launched besides the GEMV: every call leaves the slots it used empty
 * (zero) again.  Calls that overlap in time on one device share that array
 * and race: run them on one stream, or order them.  Arguments as lw_gemv.
 * Errors: as lw_gemv; LW_E_UNSUPPORTED when the bundle's reduction needs more
 * scratch than 16 MiB ((groups - 1) * 16 * rows * 4 bytes of pair slots;
 * lw_bundle_info.region_bytes[LW_REG_WORK] gives it). */
lw_status lw_gemv_noalloc(const lw_dev_bundle *db, const void *x, float *y, int batch, void *stream);

/* Decode only: restore the fixed-width codes ("3 . Decode on demand": the unit
 * restores the packed codes).
 *   Q4  : out [rows][cols/2] bytes, low nibble = even column (the twin layout)
 *   Q6  : out [rows][cols] bytes, one code each
 *   BF16: out [rows][cols] u16, the reconstructed bf16 weights
 *   lane_bits: optional device u32 [n_tiles*32] receiving each lane's consumed
 *              bit count (NULL to skip)
 * Errors: LW_E_ARG (null, out_bytes too small), LW_E_DEVICE. */
lw_status lw_decode_only(const lw_dev_bundle *db, void *out, size_t out_bytes, uint32_t *lane_bits,
                         void *stream);

/* GEMV over the fixed-width twin (ablation and latency bar).
 *   twin : device packed codes as produced by lw_twin_build
 *   dm   : device [rows][cols/256] u32
 *   x    : device fp16 [batch][cols]; y: device fp32 [batch][rows], overwritten
 * Errors: LW_E_ARG, LW_E_SHAPE, LW_E_DEVICE. */
lw_status lw_twin_gemv(const void *twin, const uint32_t *dm, int bits, int64_t rows, int64_t cols,
                       const void *x, float *y, int batch, void *stream);

/* Tile-transposed fixed-width packing for lw_skip_gemv ("Software-Defined
 * Bandwidth Expansion", IV-A storage: floor(32/b) b-bit codes per 32-bit word,
 * b in {2, 4, 8}, the lowest column in the lowest bits, so b = 3 and other
 * widths that waste word bits are not admitted; IV-B layout: words stored
 * neuron-contiguous, then tile-transposed to [n_tiles][WPR][B_N] with
 * B_N = 64 rows per tile and WPR = cols / (32/b) word columns).
 *   codes : host [rows][cols], one code per byte, each < 2^bits
 *   d, m  : host fp16 bits [rows][cols/256], w = d*q - m per 256 columns
 *   words : host out, rows*cols*bits/32 u32: word (t, j, r) at (t*WPR + j)*64 + r
 *   dm    : host out, rows*cols/256 u32 = d | m << 16 at (t*(cols/256) + g)*64 + r
 * Errors: LW_E_ARG (null, bits not 2/4/8, a code too wide), LW_E_SHAPE
 * (rows not a multiple of 64 or cols of 256). */
lw_status lw_skip_pack(const uint8_t *codes, int bits, int64_t rows, int64_t cols, const uint16_t *d,
                       const uint16_t *m, uint32_t *words, uint32_t *dm);

/* Tile-skipping fixed-width GEMV over a launch list ("Software-Defined
 * Bandwidth Expansion", IV-C: one program per active tile loads the packed
 * words, unpacks them in registers, applies scale and zero and accumulates
 * the product with x in one pass; an inactive tile is absent from the launch
 * grid, so it moves no weight bytes: n_active * WPR * 64 words are read).
 *   words, dm : device, as produced by lw_skip_pack (16-byte aligned)
 *   tiles     : device int32 [n_list], the launch list: tile t covers rows
 *               64t .. 64t+63; an entry outside 0 .. rows/64 - 1 names no
 *               tile and is skipped; a repeated entry writes the same rows
 *               again with the same values
 *   x         : device fp16 [batch][cols], 16-byte aligned
 *   y         : device fp32 [batch][rows]; only the rows of listed tiles are
 *               written, every other row keeps its contents
 *   1 <= batch <= 4 (four rows and four batch rows of partial sums stay in
 *   registers per thread); n_list = 0 enqueues nothing (pointers may then be null)
 * Each workgroup stages x in LDS: 2 * cols * batch bytes must fit in the
 * device's LDS per workgroup (LW_E_UNSUPPORTED otherwise).
 * Errors: LW_E_ARG, LW_E_SHAPE, LW_E_UNSUPPORTED, LW_E_DEVICE. */
lw_status lw_skip_gemv(const uint32_t *words, const uint32_t *dm, int bits, int64_t rows, int64_t cols,
                       const int32_t *tiles, int64_t n_list, const void *x, float *y, int batch, void *stream);

/* rANS twin of a quantised matrix: the decode-cost ablation beside the
 * Huffman lane decoder ("LazyWeights", section "Decoder hardware", where
 * Huffman and rANS decoders are compared at equal rate).  The pages fix no
 * rANS format; this one keeps the tile and symbol conventions of the Huffman
 * bundle:
 *   - one frequency table per matrix, f summing to 2^11 (absent symbols 0,
 *     present ones at least 1: each its share rounded half up, then the
 *     largest entries moved by one, ties to the smaller symbol, until the
 *     sum is exact);
 *   - one stream per tile row (halves = 1: 64 per 64x256 tile) or two
 *     (halves = 2: 128, stream h*64 + r holding half h of row r's columns):
 *     128 pair symbols a row (Q4, low nibble the even column) or 256 single
 *     codes (Q6) in column order; 32-bit state in [2^16, 2^32),
 *     renormalised 16 bits at a time;
 *   - tile t's block at word tile_off[t] with ns = 64*halves streams: the ns
 *     final encoder states (word s for stream s), then the chunks in
 *     decoding order as 16-bit units, chunk k of stream s at unit ns*k + s
 *     (little-endian halves of the following words), zero-padded to the
 *     tile's chunk count rounded up to even; a block is ns + (ns/2)k words.
 *   kind  : LW_Q4_PAIR or LW_Q6_SINGLE; codes: host [rows][cols], one code a byte
 *   halves: 1 or 2
 *   freq  : host out u16 [256] (Q4) or [64] (Q6)
 *   lut   : host out u32 [4096], derived for the kernel: slot s -> the pair
 *           (f | symbol << 24, s - cum) at [2s], [2s + 1]
 *   tile_off: host out u32 [n_tiles + 1], n_tiles = (rows/64) * (cols/256)
 *   words : host out u32 [words_cap], or NULL for a sizing pass
 *   n_words, max_tile_words: out, total words and the largest block
 * Errors: LW_E_ARG (null, bad kind, a code out of range, words_cap too
 * small), LW_E_SHAPE (shape, or offsets beyond 32 bits), LW_E_TABLE. */
lw_status lw_rans_build(int kind, int64_t rows, int64_t cols, const uint8_t *codes, int halves, uint16_t *freq,
                        uint32_t *lut, uint32_t *tile_off, uint32_t *words, int64_t words_cap, int64_t *n_words,
                        int32_t *max_tile_words);

/* Decode-only over the rANS twin (one wavefront per tile, one row per lane:
 * its one stream, or its two interleaved), writing the fixed-width codes as
 * lw_decode_only does:
 *   Q4: out [rows][cols/2] bytes, low nibble = even column; Q6: [rows][cols] bytes.
 *   lut, tile_off, words: device copies of lw_rans_build's outputs (lut,
 *   words and out 16-byte aligned); halves and max_tile_words as given to
 *   and by lw_rans_build.
 *   final_state: optional device u32 [n_tiles * 64 * halves] receiving each stream's
 *   state after its last symbol (2^16 for a well-formed stream), or NULL.
 * A block whose size does not fit max_tile_words is skipped (its output is
 * left as it was); a corrupt stream yields wrong codes and a final state
 * other than 2^16 but reads only its own block.
 * Errors: LW_E_ARG, LW_E_SHAPE, LW_E_UNSUPPORTED (blocks exceed the LDS),
 * LW_E_DEVICE. */
lw_status lw_rans_decode(int kind, int64_t rows, int64_t cols, int halves, const uint32_t *lut,
                         const uint32_t *tile_off, const uint32_t *words, int32_t max_tile_words, void *out,
                         size_t out_bytes, uint32_t *final_state, void *stream);

/* SwiGLU activation between the coded gate/up projections and the coded down
 * projection of an MLP ("Unweight", section "Overlapping Work Across
 * Transformer Layers": the down projection consumes gate, activation and up;
 * section "Measured Results": SwiGLU architectures).
 *   gate, up : device fp32 [n], e.g. the [batch][rows] outputs of lw_gemv on
 *              the gate and up bundles
 *   h        : device fp16 [n], overwritten with
 *              h = fp16_rne(silu(gate) * up),  silu(z) = z / (1 + e^-z),
 *              evaluated in fp32; the x of lw_gemv on the down bundle
 *   n        : element count (0 does nothing and accepts null pointers)
 * Enqueue-only on `stream`; any alignment (16-byte aligned buffers and n a
 * multiple of 4 take the vector path).
 * Errors: LW_E_ARG (n < 0, or a null pointer with n > 0), LW_E_DEVICE. */
lw_status lw_swiglu(const float *gate, const float *up, uint16_t *h, int64_t n, void *stream);

/* ---------------------------------------------------------------- pipelines */
/* "Unweight", sections "Four approaches to using compressed weights" and
 * "Why no single pipeline wins": full decode rebuilds every bf16 weight in
 * memory and then runs a library GEMM on it (most bytes written, the plainest
 * GEMM); the fused kernels never write the weights.  Which wins depends on
 * the batch and the matrix, so a table per uploaded bundle (filled by
 * measurement, lw_autotune) picks the pipeline of each batch bucket
 * (2^(k-1), 2^k].  Default: fused wherever it exists (batch <= 16), else
 * full decode. */

/* y = W x through full decode: lw_decode_only into wbuf (bf16 [rows][cols],
 * exact), then rocBLAS gemm_ex (bf16 x bf16, fp32 accumulate and output).
 *   wbuf : device, >= rows*cols*2 bytes, 16-byte aligned, caller-owned
 *   x    : device bf16 [batch][cols]; y: device fp32 [batch][rows]
 *   1 <= batch <= 65536; bf16 bundles only (LW_E_UNSUPPORTED otherwise:
 *   decoded 4- or 6-bit weights would be rounded)
 * The library GEMM keeps one rocBLAS handle per thread and device (with
 * rocBLAS's own workspace), created on first use: the one place where device
 * memory is allocated on the library's behalf.
 * Errors: LW_E_ARG, LW_E_UNSUPPORTED, LW_E_SHAPE, LW_E_DEVICE. */
lw_status lw_gemm_full_decode(const lw_dev_bundle *db, void *wbuf, size_t wbuf_bytes, const void *x, float *y,
                              int batch, void *stream);

/* Transcode a bf16 bundle's coded exponents into a compact form for the
 * reconstructive GEMM ("Unweight", "Four approaches to using compressed
 * weights": the exponent-only decode and the runtime palette transcode,
 * which write one byte or half a byte per weight where full decode writes
 * two).  The bundle's lane decoder
 * runs unchanged; the form is laid out tile-major, word (t, g, r) at
 * t*G*64 + g*64 + r for tile t, column group g and tile row r:
 *   LW_FORM_PALETTE : G = 32 groups of 8 columns, 8 indices a word, the
 *                     lowest column in the low nibble; rows*cols/2 bytes
 *   LW_FORM_EXPONENT: G = 64 groups of 4 columns, 4 exponent bytes a word,
 *                     the lowest column in the low byte; rows*cols bytes
 * Weights of a verbatim segment carry the placeholder (palette index 0).
 *   vrank: device int32 [n_tiles][4][64]: entry (t, s, r) = the index in the
 *          bundle's verbatim store of segment s of tile row r, or -1;
 *          n_tiles*1024 bytes
 * out and vrank 16-byte aligned.  Errors: LW_E_ARG, LW_E_UNSUPPORTED (not
 * a bf16 bundle), LW_E_DEVICE. */
lw_status lw_bf16_transcode(const lw_dev_bundle *db, int form, void *out, size_t out_bytes, int32_t *vrank,
                            size_t vrank_bytes, void *stream);

/* Reconstructive GEMM ("Unweight", "How reconstructive matmul works"):
 * y = W x for batch columns of x, the bf16 weights rebuilt on chip from
 * the form `src` (lw_bf16_transcode's layout; src_bytes and vrank_bytes at
 * least the sizes lw_bf16_transcode needs), the bundle's sign+mantissa
 * bytes and, where vrank names one, a verbatim segment's stored values, and
 * fed to the matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
 *   x: device bf16 [batch][cols]; y: device fp32 [batch][rows], overwritten
 *   1 <= batch <= 65536; variant 0..LW_RECON_VARIANTS-1, or -1 for one
 *   chosen by batch.  src, x, y 16-byte aligned, vrank 4-byte aligned.
 *   work/work_bytes: optional device scratch (16-byte aligned) for partial
 *   sums: when the grid would be short of wavefronts, the column blocks are
 *   split up to 8 ways (as far as splits * batch * rows * 4 bytes fit) and
 *   a second kernel adds the partials in split order.
 * The sums run in a fixed order: results are deterministic.
 * Errors: LW_E_ARG, LW_E_UNSUPPORTED, LW_E_DEVICE. */
lw_status lw_recon_gemm(const lw_dev_bundle *db, int form, const void *src, size_t src_bytes, const int32_t *vrank,
                        size_t vrank_bytes, const void *x, float *y, int batch, int variant, void *work,
                        size_t work_bytes, void *stream);

/* Transcode the bundle into the palette form once ("Unweight": the direct
 * palette pipeline, whose weights are transcoded at load time) into `buf`
 * (device, 256-byte aligned, at least lw_pipeline_scratch_bytes(db,
 * LW_PIPE_DIRECT_PALETTE) bytes, caller-owned and kept alive while the
 * bundle is used) and keep it with the bundle for LW_PIPE_DIRECT_PALETTE.
 * Errors: LW_E_ARG, LW_E_UNSUPPORTED, LW_E_DEVICE. */
lw_status lw_bundle_attach_palette(lw_dev_bundle *db, void *buf, size_t bytes, void *stream);

/* Bytes of caller scratch (wbuf of lw_gemm and lw_autotune) a pipeline needs
 * on this bundle (0 for the fused pipeline), or for LW_PIPE_DIRECT_PALETTE
 * the size of lw_bundle_attach_palette's buffer. */
size_t lw_pipeline_scratch_bytes(const lw_dev_bundle *db, int pipeline);

/* Set the pipeline (lw_pipeline) of the buckets holding batch_lo..batch_hi.
 * Errors: LW_E_ARG, LW_E_UNSUPPORTED (the pipeline does not serve that batch
 * or bundle kind). */
lw_status lw_pipeline_set(lw_dev_bundle *db, int batch_lo, int batch_hi, int pipeline);
lw_status lw_pipeline_get(const lw_dev_bundle *db, int batch, int *pipeline);

/* y = W x through the pipeline the bundle's table names for this batch (and,
 * for the reconstructive pipelines, the variant the autotuner chose there).
 * wbuf/wbuf_bytes is the caller's scratch for full decode, the exponent-only
 * and the palette pipelines (lw_pipeline_scratch_bytes; 256-byte aligned
 * for the latter two; may be NULL/0 while the table picks the fused or the
 * direct palette pipeline).  Errors: as the pipelines'. */
lw_status lw_gemm(const lw_dev_bundle *db, const void *x, float *y, int batch, void *wbuf, size_t wbuf_bytes,
                  void *stream);

/* Measure every available pipeline at each of the n batch sizes (one warm-up
 * call, then `reps` timed calls between HIP events on `stream`, synchronised
 * here; the reconstructive pipelines in each variant) and set each batch's
 * bucket to the fastest pipeline and variant ("Unweight", "Autotuning the
 * configuration space").  x and y must hold the largest batch.  us_out
 * (optional, host float [n][LW_PIPE_COUNT]) receives the microseconds per
 * call (the best variant's), -1 where a pipeline does not apply.  A pipeline
 * whose scratch does not fit wbuf is left out (wbuf = NULL: all of them but
 * the fused and the direct palette pipelines).
 * Errors: LW_E_ARG and those of the pipelines. */
lw_status lw_autotune(lw_dev_bundle *db, const int *batches, int n, void *wbuf, size_t wbuf_bytes, const void *x,
                      float *y, int reps, void *stream, float *us_out);

/* ---------------------------------------------------------------- measurement */

/* Read-only streaming probe: reads `bytes` from device memory `src` with
 * fully coalesced 16-byte loads (512 threads per workgroup, eight loads per
 * thread, all issued before use) and writes nothing except, to keep the loads
 * live, sink[0] when the XOR of a thread's words equals 0x9E3779B9.  Timed
 * beside the decoding kernels, it gives the HBM bandwidth a kernel that only
 * reads attains at a given size (context for their fraction of peak; not part
 * of the decode path).
 *   src : device, 16-byte aligned; bytes: a positive multiple of 16
 *   sink: device u32, 4-byte aligned
 * Errors: LW_E_ARG, LW_E_DEVICE. */
lw_status lw_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream);

const char *lw_status_str(lw_status s);
const char *lw_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LW_H */
