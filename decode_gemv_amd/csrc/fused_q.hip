// fused_q.hip -- fused decode + dequantise + GEMV (batch 1..7, VALU) and
// decode-only kernels for 4-bit pair and 6-bit single codes, gfx950.
//
// Work split ("LazyWeights", section "2 . Code them": a 64x256 tile is 32
// lanes of two rows): one wavefront decodes two tiles of the same column
// block -- lanes 0..31 row band 2p, lanes 32..63 row band 2p+1 -- so every
// lane of the wavefront consumes the same activation pair at each step and x
// is read once per wavefront from LDS.  A workgroup of four wavefronts covers
// four consecutive column blocks of one row-band pair; workgroups of different
// column groups are combined by a fixed-order reduction through the bundle's
// workspace (the last workgroup to arrive sums the partials in group order),
// so the result is deterministic.
//
// Dequantisation w = d*q - m per 256-weight super-block (one tile row) is
// applied after the dot product: y = d * sum(q x) - m * sum(x).
#include "kernels.h"
#include "lane_decode.hpp"

namespace {

constexpr int WAVES = 4;

LW_DEV int slots_of(int max_words) { return max_words + 2; }

struct LdsLayout {
    size_t tab, x, tiles, total;
};

__host__ __device__ inline LdsLayout lds_layout(int batch, int max_words, bool decode_only)
{
    LdsLayout L;
    L.tab = 0;
    L.x = (sizeof(LdsTab) + 255) & ~(size_t)255;
    size_t xbytes = decode_only ? 0 : (size_t)WAVES * batch * 128 * 4;
    L.tiles = L.x + xbytes;
    size_t tiles = (size_t)WAVES * 2 * (max_words + 2) * 128;
    size_t red = (size_t)WAVES * batch * 128 * 4;
    L.total = L.tiles + (tiles > red ? tiles : red);
    return L;
}

// Shared prologue: tables, this wave's two tiles, and the lane's identity.
struct LaneCtx {
    int wave, lane, half, l, g, rbp, cb, rb, t;
    bool wave_active, lane_active;
};

LW_DEV LaneCtx lane_ctx(const KArgs &a)
{
    LaneCtx c;
    c.wave = (int)lw_wave_id();
    c.lane = threadIdx.x & 63;
    c.half = c.lane >> 5;
    c.l = c.lane & 31;
    c.g = blockIdx.x;
    c.rbp = blockIdx.y;
    c.cb = c.g * WAVES + c.wave;
    c.wave_active = c.cb < a.n_cb;
    int rb = c.rbp * 2 + c.half;
    c.lane_active = c.wave_active && rb < a.n_rb;
    // a missing second row band decodes the first one again; its results are dropped
    c.rb = rb < a.n_rb ? rb : rb - 1;
    c.t = c.rb * a.n_cb + (c.wave_active ? c.cb : 0);
    return c;
}

template <int KIND, int NCMP, int BATCH>
__global__ __launch_bounds__(256) void k_gemv_q(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int SPL = KIND == LW_Q4_PAIR ? 256 : 512;
    const LdsLayout L = lds_layout(BATCH, a.max_words, false);
    LdsTab &tab = *reinterpret_cast<LdsTab *>(lds + L.tab);
    const LaneCtx c = lane_ctx(a);
    const int S = slots_of(a.max_words);
    uint32_t *xs = reinterpret_cast<uint32_t *>(lds + L.x) + c.wave * BATCH * 128;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + (c.wave * 2 + c.half) * S * 32;

    lw_stage_tab(tab, a.tab, false);
    float sx[BATCH];
    if (c.wave_active) {
        const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
        lw_stage_tile(slots, a.words, w0, (w1 - w0) >> 5, c.l);
        const uint32_t *xg = reinterpret_cast<const uint32_t *>(a.x);
#pragma unroll
        for (int b = 0; b < BATCH; b++) {
            const uint32_t *xb = xg + (size_t)b * (a.cols / 2) + (size_t)c.cb * 128;
            uint32_t v0 = xb[c.lane], v1 = xb[c.lane + 64];
            xs[b * 128 + c.lane] = v0;
            xs[b * 128 + c.lane + 64] = v1;
            sx[b] = lw_wave_sum(lw_half_lo(v0) + lw_half_hi(v0) + lw_half_lo(v1) + lw_half_hi(v1));
        }
    }
    __syncthreads();

    float acc[2][BATCH];
#pragma unroll
    for (int p = 0; p < 2; p++)
#pragma unroll
        for (int b = 0; b < BATCH; b++) acc[p][b] = 0.f;

    if (c.wave_active) {
        const uint32_t *lw = slots + c.l;
        uint32_t u = 31;
#pragma unroll
        for (int p = 0; p < 2; p++) {
#pragma unroll 4
            for (int k = 0; k < SPL / 2; k++) {
                const uint32_t idx = lw_decode_step<NCMP>(lw, u, a.lim, tab);
                if constexpr (KIND == LW_Q4_PAIR) {
                    const uint32_t pay = tab.pay[idx];
#pragma unroll
                    for (int b = 0; b < BATCH; b++) acc[p][b] = lw_dot2(pay, xs[b * 128 + k], acc[p][b]);
                } else {
                    const uint32_t pay = (k & 1) ? tab.pay_hi[idx] : tab.pay[idx];
#pragma unroll
                    for (int b = 0; b < BATCH; b++) acc[p][b] = lw_dot2(pay, xs[b * 128 + (k >> 1)], acc[p][b]);
                }
            }
        }
    }

    // dequantise: y_row = d * sum(q x) - m * sum(x) for this tile row
    float val[2][BATCH];
    if (c.wave_active) {
        const uint2 dm = *reinterpret_cast<const uint2 *>(a.dm + (size_t)c.t * 64 + 2 * c.l);
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const uint32_t w = p ? dm.y : dm.x;
            const float d = lw_half_lo(w), m = lw_half_hi(w);
#pragma unroll
            for (int b = 0; b < BATCH; b++) val[p][b] = d * acc[p][b] - m * sx[b];
        }
    }
    __syncthreads();                      // tiles no longer read: reuse for the reduction
    float *red = reinterpret_cast<float *>(lds + L.tiles);
    // red[wave][b][row], row = half*64 + 2l + p within the workgroup's 128 rows
#pragma unroll
    for (int p = 0; p < 2; p++)
#pragma unroll
        for (int b = 0; b < BATCH; b++)
            red[(c.wave * BATCH + b) * 128 + c.half * 64 + 2 * c.l + p] =
                (c.wave_active && c.lane_active) ? val[p][b] : 0.f;
    __syncthreads();

    const int64_t row0 = (int64_t)c.rbp * 128;
    __shared__ uint32_t last_flag;
    for (int i = threadIdx.x; i < BATCH * 128; i += blockDim.x) {
        const int b = i >> 7, row = i & 127;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; w++) v += red[(w * BATCH + b) * 128 + row];
        if (row0 + row < a.rows) {
            if (a.groups == 1) a.y[(size_t)b * a.rows + row0 + row] = v;
            else a.part[((size_t)c.g * LW_BATCH_MAX + b) * a.rows + row0 + row] = v;
        }
    }
    if (a.groups == 1) return;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = atomicAdd(&a.count[c.rbp], 1u);
        last_flag = (old == (uint32_t)a.groups - 1u) ? 1u : 0u;
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    for (int i = threadIdx.x; i < BATCH * 128; i += blockDim.x) {
        const int b = i >> 7, row = i & 127;
        if (row0 + row >= a.rows) continue;
        float v = 0.f;
        for (int g = 0; g < a.groups; g++)
            v += __builtin_nontemporal_load(&a.part[((size_t)g * LW_BATCH_MAX + b) * a.rows + row0 + row]);
        a.y[(size_t)b * a.rows + row0 + row] = v;
    }
    if (threadIdx.x == 0) a.count[c.rbp] = 0u;
}

// Decode only: restore the fixed-width codes (Q4 packed nibbles, Q6 bytes).
template <int KIND, int NCMP>
__global__ __launch_bounds__(256) void k_decode_q(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int SPL = KIND == LW_Q4_PAIR ? 256 : 512;
    const LdsLayout L = lds_layout(1, a.max_words, true);
    LdsTab &tab = *reinterpret_cast<LdsTab *>(lds + L.tab);
    const LaneCtx c = lane_ctx(a);
    const int S = slots_of(a.max_words);
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + (c.wave * 2 + c.half) * S * 32;
    lw_stage_tab(tab, a.tab, true);
    if (c.wave_active) {
        const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
        lw_stage_tile(slots, a.words, w0, (w1 - w0) >> 5, c.l);
    }
    __syncthreads();
    if (!c.wave_active) return;
    const uint32_t *lw = slots + c.l;
    uint32_t u = 31;
    uint32_t *out = reinterpret_cast<uint32_t *>(a.out);
    const int64_t row_bytes = KIND == LW_Q4_PAIR ? a.cols / 2 : a.cols;
#pragma unroll
    for (int p = 0; p < 2; p++) {
        const int64_t row = (int64_t)c.rb * 64 + 2 * c.l + p;
        uint32_t *orow = out + (row * row_bytes + (int64_t)c.cb * (SPL / 2)) / 4;
        uint32_t pk = 0;
#pragma unroll 4
        for (int k = 0; k < SPL / 2; k++) {
            const uint32_t idx = lw_decode_step<NCMP>(lw, u, a.lim, tab);
            pk |= tab.pay_hi[idx] << (8 * (k & 3));
            if ((k & 3) == 3) {
                if (c.lane_active) orow[k >> 2] = pk;
                pk = 0;
            }
        }
    }
    if (a.lane_bits && c.lane_active) a.lane_bits[(size_t)c.t * 32 + c.l] = u - 31;
}

template <int KIND, int NCMP, int BATCH>
hipError_t launch_gemv_q(const KArgs &a, hipStream_t s)
{
    const LdsLayout L = lds_layout(BATCH, a.max_words, false);
    dim3 grid((unsigned)a.groups, (unsigned)((a.n_rb + 1) / 2));
    auto kern = k_gemv_q<KIND, NCMP, BATCH>;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.total);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(256), L.total, s, a);
    return hipGetLastError();
}

template <int KIND, int NCMP>
hipError_t launch_decode_q(const KArgs &a, hipStream_t s)
{
    const LdsLayout L = lds_layout(1, a.max_words, true);
    dim3 grid((unsigned)a.groups, (unsigned)((a.n_rb + 1) / 2));
    auto kern = k_decode_q<KIND, NCMP>;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.total);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(256), L.total, s, a);
    return hipGetLastError();
}

template <int KIND, int NCMP>
hipError_t gemv_batch(const KArgs &a, int batch, hipStream_t s)
{
    switch (batch) {
    case 1: return launch_gemv_q<KIND, NCMP, 1>(a, s);
    case 2: return launch_gemv_q<KIND, NCMP, 2>(a, s);
    case 3: return launch_gemv_q<KIND, NCMP, 3>(a, s);
    case 4: return launch_gemv_q<KIND, NCMP, 4>(a, s);
    case 5: return launch_gemv_q<KIND, NCMP, 5>(a, s);
    case 6: return launch_gemv_q<KIND, NCMP, 6>(a, s);
    case 7: return launch_gemv_q<KIND, NCMP, 7>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int KIND>
hipError_t gemv_ncmp(const KArgs &a, int ncmp, int batch, hipStream_t s)
{
    switch (ncmp) {
    case 0: return gemv_batch<KIND, 0>(a, batch, s);
    case 1: return gemv_batch<KIND, 1>(a, batch, s);
    case 2: return gemv_batch<KIND, 2>(a, batch, s);
    case 3: return gemv_batch<KIND, 3>(a, batch, s);
    case 4: return gemv_batch<KIND, 4>(a, batch, s);
    case 5: return gemv_batch<KIND, 5>(a, batch, s);
    case 6: return gemv_batch<KIND, 6>(a, batch, s);
    case 7: return gemv_batch<KIND, 7>(a, batch, s);
    case 8: return gemv_batch<KIND, 8>(a, batch, s);
    case 9: return gemv_batch<KIND, 9>(a, batch, s);
    case 10: return gemv_batch<KIND, 10>(a, batch, s);
    }
    return hipErrorInvalidValue;
}

template <int KIND>
hipError_t decode_ncmp(const KArgs &a, int ncmp, hipStream_t s)
{
    switch (ncmp) {
    case 0: return launch_decode_q<KIND, 0>(a, s);
    case 1: return launch_decode_q<KIND, 1>(a, s);
    case 2: return launch_decode_q<KIND, 2>(a, s);
    case 3: return launch_decode_q<KIND, 3>(a, s);
    case 4: return launch_decode_q<KIND, 4>(a, s);
    case 5: return launch_decode_q<KIND, 5>(a, s);
    case 6: return launch_decode_q<KIND, 6>(a, s);
    case 7: return launch_decode_q<KIND, 7>(a, s);
    case 8: return launch_decode_q<KIND, 8>(a, s);
    case 9: return launch_decode_q<KIND, 9>(a, s);
    case 10: return launch_decode_q<KIND, 10>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t lw_lds_bytes(int kind, int batch, int max_words, bool decode_only)
{
    (void)kind;
    return lds_layout(batch, max_words, decode_only).total;
}

hipError_t lw_launch_gemv_q(const KArgs &a, int kind, int ncmp, int batch, hipStream_t s)
{
    if (kind == LW_Q4_PAIR) return gemv_ncmp<LW_Q4_PAIR>(a, ncmp, batch, s);
    if (kind == LW_Q6_SINGLE) return gemv_ncmp<LW_Q6_SINGLE>(a, ncmp, batch, s);
    return hipErrorInvalidValue;
}

hipError_t lw_launch_decode_q(const KArgs &a, int kind, int ncmp, hipStream_t s)
{
    if (kind == LW_Q4_PAIR) return decode_ncmp<LW_Q4_PAIR>(a, ncmp, s);
    if (kind == LW_Q6_SINGLE) return decode_ncmp<LW_Q6_SINGLE>(a, ncmp, s);
    return hipErrorInvalidValue;
}
