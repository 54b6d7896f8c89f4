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
    int64_t rows, cols;
    int32_t n_rb, n_cb, groups, batch, max_words, min_len;
    uint32_t pal0;               // bf16: exponent of palette index 0
    uint32_t lim[10];            // left-justified limits for lengths min_len .. max_len-1
};

// LDS bytes a fused/decode kernel needs per workgroup
size_t lw_lds_bytes(int kind, int batch, int max_words, bool decode_only);

hipError_t lw_launch_gemv_q(const KArgs &a, int kind, int ncmp, int batch, hipStream_t s);
hipError_t lw_launch_decode_q(const KArgs &a, int kind, int ncmp, hipStream_t s);
hipError_t lw_launch_gemv_mfma(const KArgs &a, int kind, int ncmp, int batch, hipStream_t s);
hipError_t lw_launch_gemv_bf16(const KArgs &a, int ncmp, int batch, hipStream_t s);
hipError_t lw_launch_decode_bf16(const KArgs &a, int ncmp, hipStream_t s);
hipError_t lw_launch_twin(const uint8_t *twin, const uint32_t *dm, int64_t rows, int64_t cols,
                          const uint16_t *x, float *y, int batch, hipStream_t s);
hipError_t lw_launch_fill_zero(void *p, size_t bytes, hipStream_t s);

#endif
