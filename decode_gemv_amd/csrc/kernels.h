// kernels.h -- launch interface between the runtime (runtime.hip) and the
// gfx950 kernels of liblw.  Internal to the library.
#ifndef LW_KERNELS_H
#define LW_KERNELS_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lw_internal.h"

// Everything a kernel needs about one uploaded bundle and one call.  Passed
// by value: scalars and the limit registers land in SGPRs.
struct KArgs {
    const uint32_t *words;       // interleaved lane words
    const uint32_t *tile_off;    // [n_tiles+1]
    const uint16_t *split;       // [n_tiles][32] first bit of each lane's second tile row
    const uint32_t *dm;          // [n_tiles][64] d | m << 16 (Q4/Q6)
    const lw_gputab *tab;        // derived tables
    const uint32_t *sm;          // bf16 sign+mantissa words
    const uint32_t *vb_bits;     // bf16 verbatim bitmap
    const uint32_t *vb_start;    // bf16 verbatim ordinal of each tile
    const uint16_t *verbatim;    // bf16 raw segments
    const uint16_t *x;           // [batch][cols] fp16 or bf16 bits
    float *y;                    // [batch][rows]
    float *part;                 // workspace partials [groups][16][rows]
    uint32_t *count;             // workspace arrival counters
    void *out;                   // decode-only output
    uint32_t *lane_bits;         // decode-only optional per-lane bit counts
    int32_t *vrank;              // bf16 transcode: verbatim store index of each (tile, segment, row), or -1
    int64_t rows, cols;
    int32_t n_rb, n_cb, groups, batch, max_words, min_len, max_len;
    uint32_t pal0;               // bf16: exponent of palette index 0
    // Limit comparison by sums of absolute differences (see lane_decode.hpp):
    // byte lanes compare the top 8 peek bits with limit/8 (lengths <= 8),
    // 16-bit lanes the top 16 window bits with limit*32 (lengths 9, 10).
    uint32_t c8[2], c8m1[2];     // limit/8 and limit/8 - 1 per byte, 0 in unused bytes
    uint32_t c16, c16m1;         // limit*32 and limit*32 - 1 per half, 0 in unused halves
    uint32_t sad_k;              // accumulator offset: PBASE - 2*min_len - (number of comparisons)
    // Compact tables (at most four code lengths, the three shorter <= 8): the
    // comparison count r indexes the used lengths; lut_hi:lut_lo hold
    // -length(r) mod 256 at byte 7 - 2r and 0xFF in the even bytes,
    // cbase[r] = offset - first of length(r)
    uint32_t lut_lo, lut_hi;
    int32_t cbase[4];
    int32_t ncmp;                // comparisons (used lengths - 1)
    int32_t ramp;                // 1: the whole grid is resident at once (wavefronts lower their priority as they progress)
};

// SAD comparison layout of a bundle: byte-lane ops (0..2) and 16-bit ops
// (0..1); compact tables use one byte-lane op and the count-indexed tables
// (kernels instantiate them with N16 == LW_N16_COMPACT)
struct SadPlan {
    int n8ops, n16ops;
    bool compact;
};
#define LW_N16_COMPACT 2
SadPlan lw_sad_plan(const lw_table &t, int min_len, int max_len, KArgs &a);

// LDS bytes a fused/decode kernel needs per workgroup

hipError_t lw_launch_gemv_q(const KArgs &a, int kind, SadPlan p, int batch, hipStream_t s);
hipError_t lw_launch_decode_q(const KArgs &a, int kind, SadPlan p, hipStream_t s);
hipError_t lw_launch_gemv_mfma(const KArgs &a, int kind, SadPlan p, int batch, hipStream_t s);
hipError_t lw_launch_gemv_bf16(const KArgs &a, SadPlan p, int batch, hipStream_t s);
hipError_t lw_launch_decode_bf16(const KArgs &a, SadPlan p, hipStream_t s);
hipError_t lw_launch_transcode_bf16(const KArgs &a, SadPlan p, bool exponents, hipStream_t s);
hipError_t lw_launch_swiglu(const float *g, const float *u, uint16_t *h, int64_t n, hipStream_t s);
hipError_t lw_launch_twin(const uint8_t *twin, const uint32_t *dm, int64_t rows, int64_t cols,
                          const uint16_t *x, float *y, int batch, hipStream_t s);
hipError_t lw_launch_fill_zero(void *p, size_t bytes, hipStream_t s);
hipError_t lw_launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s);
hipError_t lw_launch_recon(bool exponents, const uint32_t *src, const uint32_t *sm, const int32_t *vrank,
                           const uint32_t *vb_start, const uint16_t *verbatim, int64_t n_verbatim,
                           const uint8_t *palette, const uint16_t *x, float *y, int64_t rows, int64_t cols,
                           int batch, int variant, float *part, int splits, hipStream_t s);
hipError_t lw_launch_rans_decode(int spr, int halves, const uint32_t *lut, const uint32_t *tile_off,
                                 const uint32_t *words, uint8_t *out, uint32_t *final_state, int64_t nt, int ncb,
                                 int64_t out_stride, int max_tile_words, hipStream_t s);
hipError_t lw_launch_skip(const uint32_t *words, const uint32_t *dm, int bits, int64_t rows, int64_t cols,
                          const int32_t *tiles, int64_t n_list, const uint16_t *x, float *y, int batch,
                          hipStream_t s);

#endif
