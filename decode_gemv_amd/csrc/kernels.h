// kernels.h -- launch interface between the runtime (runtime.hip) and the
// gfx950 kernels of liblw.  Internal to the library.
#ifndef LW_KERNELS_H
#define LW_KERNELS_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lw_internal.h"

// Everything a kernel needs about one uploaded bundle and one call.  Passed
// by value: scalars and the limit registers land in SGPRs.
struct KArgs {
    const uint32_t *words;       // interleaved lane words
    const uint32_t *tile_off;    // [n_tiles+1]
    const uint16_t *split;       // [n_tiles][2*parts-1][32] first bit of each part of a lane stream
    const uint32_t *dm;          // [n_tiles][64] d | m << 16 (Q4/Q6)
    const lw_gputab *tab;        // derived tables
    const uint32_t *sm;          // bf16 sign+mantissa words
    const uint32_t *vb_bits;     // bf16 verbatim bitmap
    const uint32_t *vb_start;    // bf16 verbatim ordinal of each tile
    const uint16_t *verbatim;    // bf16 raw segments
    const uint16_t *x;           // [batch][cols] fp16 or bf16 bits
    float *y;                    // [batch][rows]
    float *part;                 // workspace: pair slots of the reduction tree [groups-1][16][rows]
    void *out;                   // decode-only output
    uint32_t *lane_bits;         // decode-only optional per-lane bit counts
    int32_t *vrank;              // bf16 transcode: verbatim store index of each (tile, segment, row), or -1
    int64_t rows, cols;
    int32_t n_rb, n_cb, groups, batch, max_words, min_len, max_len;
    int32_t parts;               // parts per tile row with a recorded start (1, 2, 4 or 8)
    uint32_t pal0;               // bf16: exponent of palette index 0
    // Limit comparison by sums of absolute differences (see lane_decode.hpp).
    // c8[j], c8m1[j]: the byte thresholds of SAD pair j (t and t - 1 per
    // byte, equal in unused bytes).  Residue plans: byte i of the compared
    // register X is the top peek byte (xsel byte 3) or the top byte of the
    // peek plus xk[.] (saturating; xsel byte 7), so a limit that is not a
    // multiple of 8 is compared exactly too.  General plan: c16, c16m1 hold
    // limit*32 (and - 1) per half for lengths 9 and 10 on the top 16 bits.
    uint32_t c8[2], c8m1[2];
    uint32_t c16, c16m1;
    uint32_t xsel[2], xk[2];
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

// Comparison plans of the lane decoder (lane_decode.hpp, lw_count):
//   LW_P_COMPACT  at most four used lengths, the three shorter <= 8: one SAD
//                 pair on the replicated top peek byte, length from a byte table
//   LW_P_R2       every limit a multiple of 8, at most 8 comparisons: two SAD
//                 pairs on the replicated top peek byte, length min_len + count
//   LW_P_R2K      as R2 with one more residue: some bytes come from the peek
//                 plus a constant, so limits congruent to r mod 8 compare exactly
//   LW_P_R2X2     two residues besides 0: each SAD pair has its own register
//   LW_P_GEN      anything else (more than 8 comparisons): two byte pairs on
//                 the top byte and one 16-bit pair on the top 16 bits
//   LW_P_S2K      tables with absent lengths whose used lengths fit where the
//                 full range does not: as R2K over the used lengths only, the
//                 length of count r from a byte table indexed by A / 2
struct SadPlan {
    int plan;
};
// Copy a bundle's comparison plan into the kernel arguments.
SadPlan lw_apply_plan(const lw_plan &p, KArgs &a);

// Call f(std::integral_constant<int, PLAN>{}) for the plan's compile-time value.
template <class F>
inline hipError_t lw_with_plan(SadPlan p, F f)
{
    switch (p.plan) {
    case LW_P_COMPACT: return f(std::integral_constant<int, LW_P_COMPACT>{});
    case LW_P_R2: return f(std::integral_constant<int, LW_P_R2>{});
    case LW_P_R2K: return f(std::integral_constant<int, LW_P_R2K>{});
    case LW_P_R2X2: return f(std::integral_constant<int, LW_P_R2X2>{});
    case LW_P_GEN: return f(std::integral_constant<int, LW_P_GEN>{});
    case LW_P_S2K: return f(std::integral_constant<int, LW_P_S2K>{});
    }
    return hipErrorInvalidValue;
}

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
