/*
 * lw_internal.h -- bundle image layout shared by the host builder and the
 * device runtime of liblw (not part of the public ABI).
 *
 * An image is one little-endian byte array: a 512-byte header followed by the
 * regions of lw_region, each starting on a 256-byte boundary, so that one
 * device buffer holds a whole matrix and every region is aligned for wide
 * loads.
 */
#ifndef LW_INTERNAL_H
#define LW_INTERNAL_H

#include <stdint.h>
#include "lw.h"

#define LW_MAGIC 0x3142574Cu       /* "LWB1" */
#define LW_VERSION 4u
#define LW_MAXLEN 11               /* "LazyWeights", 2 . Code them: 11-bit codes */
#define LW_TILE_ROWS 64            /* a 64x256 tile is 32 lanes of two rows */
#define LW_TILE_COLS 256
#define LW_LANES 32
#define LW_ALIGN 256
#define LW_HEADER_BYTES 512
#define LW_BATCH_MAX 16             /* largest batch of the fused kernels */
#define LW_GEMM_BATCH_MAX 65536     /* largest batch of lw_gemm */
#define LW_CB_PER_WG 4             /* decoding units (wavefronts) of the smallest workgroup */
/* Decoding units (tiles x parts per tile row) the default part count stays
 * within: four wavefronts on each of the 1024 SIMDs of 256 compute units.
 * Measured on MI355X at batch 1, matrices of 16 to 2048 tiles run fastest
 * with the most parts that keep tiles x parts <= 4096 (e.g. 1024x4096: 6.2 us
 * in eight parts against 16.1 us in whole rows); from about 3584 tiles whole
 * rows in one part are as fast or faster, and need no extra starts. */
#define LW_PART_UNITS 4096

typedef struct {
    uint32_t magic;
    uint32_t version;
    int32_t kind;
    int32_t bits;
    int64_t rows;
    int64_t cols;
    int64_t n_tiles;
    int32_t n_rb;
    int32_t n_cb;
    int32_t spl;                   /* symbols per lane */
    int32_t n_sym;
    int32_t min_len;
    int32_t max_len;
    int32_t max_words;
    int32_t n_pal;
    int64_t n_verbatim;
    int32_t work_groups;           /* split-column groups the workspace is sized for */
    int32_t code;                  /* lw_code the lengths were chosen by */
    uint64_t coded_bytes;
    uint64_t twin_bytes;
    uint64_t off[LW_REG_COUNT];
    uint64_t bytes[LW_REG_COUNT];
    int32_t parts;                 /* parts per tile row whose starts LW_REG_SPLIT holds: 1, 2, 4 or 8 */
    int32_t reserved;
} lw_image_header;

/* LW_REG_TABLE: the canonical decoder table of the matrix. */
typedef struct {
    uint16_t count[12];
    uint16_t first[12];
    uint16_t limit[12];            /* (first + count) << (11 - L): 11-bit peek bound */
    uint16_t offset[12];
    uint16_t sym_sorted[256];
} lw_table;

/* How a lane decoder compares its peek with the limits (derived from the
 * table at build time, checked again on load).  plan is one of the kernels'
 * comparison plans (kernels.h); c8/c8m1 hold the byte thresholds t and t - 1
 * of the two SAD pairs, c16/c16m1 the 16-bit ones of the general plan, xsel
 * and xk the byte gather and additive constant of the residue plans, sad_k
 * the accumulator offset; lut_lo/lut_hi, cbase and ncmp the compact tables'
 * shift bytes and bases. */
typedef struct {
    int32_t plan;
    uint32_t sad_k;
    uint32_t c8[2], c8m1[2];
    uint32_t c16, c16m1;
    uint32_t xsel[2], xk[2];
    uint32_t lut_lo, lut_hi;
    int32_t cbase[4];
    int32_t ncmp;
    int32_t reserved[3];
} lw_plan;

/* LW_REG_GPUTAB: tables derived from lw_table for the kernels.
 * With r = number of lengths L in [min_len, max_len) whose limit is <= the
 * peek, the code length is min_len + r. */
typedef struct {
    uint32_t limlj[16];            /* limit[min_len + i] << 21, i < max_len - min_len; else ~0 */
    uint32_t len[16];              /* code length for comparison count r */
    int32_t base[16];              /* offset[len] - first[len] for comparison count r */
    uint32_t payload[256];         /* per canonical index: Q4 half2(q_even, q_odd); Q6 half2(q, 0);
                                      bf16: exponent << 7 (low bf16 of a pair) */
    uint32_t payload_hi[256];      /* Q6 half2(0, q); bf16 exponent << 23 (high bf16 of a pair) */
    uint32_t symval[256];          /* the symbol itself (decode-only) */
    lw_plan plan;                  /* the decoders' comparison plan */
} lw_gputab;

/* LDS byte offsets the plans' accumulator offsets are relative to: the
 * length entries sit at PBASE - 2*len, the compact tables' at CSEL + 1 - 2r,
 * the sparse plan's at SBASE - 2r (SBASE / 2 = 7 mod 256, so that the low
 * byte of A / 2 is the byte-table selector 7 - r). */
#define LW_PLAN_PBASE 1024u
#define LW_PLAN_CSEL 0xD07u
#define LW_PLAN_SBASE 526u

/* Comparison plans (lane_decode.hpp): see kernels.h. */
enum { LW_P_COMPACT = 0, LW_P_R2 = 1, LW_P_R2K = 2, LW_P_R2X2 = 3, LW_P_GEN = 4, LW_P_S2K = 5 };

/* Regions each kind of kernel reads (bundle.cpp): a bit mask over lw_region.
 * LW_OP_ANY is the union over every kernel of the kind (what a valid image
 * must hold); the launch paths check their own op before enqueueing. */
enum { LW_OP_GEMV = 0, LW_OP_DECODE = 1, LW_OP_ANY = 2 };
uint32_t lw_regions_needed(const lw_image_header &h, int op);
const char *lw_region_name(int r);

/* Derive the comparison plan of a canonical table (bundle.cpp). */
void lw_make_plan(const lw_table &t, int min_len, int max_len, lw_plan &p);

static inline uint64_t lw_align_up(uint64_t v) { return (v + LW_ALIGN - 1) & ~(uint64_t)(LW_ALIGN - 1); }

/* Column groups the workspace holds partials for: a row band's tiles x parts
 * over the smallest workgroup (every launch combines at most this many). */
static inline int32_t lw_work_groups(int64_t n_cb, int32_t parts)
{
    return (int32_t)((n_cb * parts + LW_CB_PER_WG - 1) / LW_CB_PER_WG);
}

/* workspace layout: the pair slots of the split-column reduction's exchange
 * tree, [groups - 1][LW_BATCH_MAX][rows] f32 (combining G groups takes G - 1
 * pair slots), all zero (empty) between calls */
static inline uint64_t lw_work_bytes(int32_t groups, int64_t rows)
{
    return groups > 1 ? (uint64_t)(groups - 1) * LW_BATCH_MAX * (uint64_t)rows * 4u : 0u;
}

#endif
