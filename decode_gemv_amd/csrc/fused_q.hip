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
#include <type_traits>

#include "lane_decode.hpp"

namespace {

constexpr int WAVES = 4;

struct LdsLayout {
    uint32_t x, tiles, flag, total;
};

__host__ __device__ inline LdsLayout lds_layout(int batch, int max_words, bool decode_only)
{
    LdsLayout L;
    L.x = LW_TAB_BYTES;
    const uint32_t xbytes = decode_only ? 0u : (uint32_t)(WAVES * batch * 128 * 4);
    L.tiles = L.x + xbytes;
    const uint32_t tiles = (uint32_t)(WAVES * 2 * (max_words + 3) * 128);
    const uint32_t red = (uint32_t)(WAVES * batch * 128 * 4);
    L.flag = L.tiles + (tiles > red ? tiles : red);
    L.total = L.flag + 16;
    return L;
}

// Identity of a lane within the grid.
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
    const int rb = c.rbp * 2 + c.half;
    c.lane_active = c.wave_active && rb < a.n_rb;
    // a missing second row band decodes the first one again; its results are dropped
    c.rb = rb < a.n_rb ? rb : rb - 1;
    c.t = c.rb * a.n_cb + (c.wave_active ? c.cb : 0);
    return c;
}

template <int KIND, int N8, int N16, int BATCH>
__global__ __launch_bounds__(256) void k_gemv_q(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int SPL = KIND == LW_Q4_PAIR ? 256 : 512;
    const LdsLayout L = lds_layout(BATCH, a.max_words, false);
    const LaneCtx c = lane_ctx(a);
    const int S = a.max_words + 3;
    uint32_t *xs = reinterpret_cast<uint32_t *>(lds + L.x) + c.wave * BATCH * 128;
    const uint32_t xs_addr = (uint32_t)(size_t)xs;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + (c.wave * 2 + c.half) * S * 32;

    lw_stage_tab(lds, a.tab, a.min_len, a.max_len, false);
    float sx[BATCH];
    uint2 dm = make_uint2(0u, 0u);       // (d, m) of this lane's two tile rows, fetched with the tile
    if (c.wave_active) {
        const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
        dm = *reinterpret_cast<const uint2 *>(a.dm + (size_t)c.t * 64 + 2 * c.l);
        lw_stage_tile(slots, a.words, w0, (w1 - w0) >> 5, c.l);
        const uint32_t *xg = reinterpret_cast<const uint32_t *>(a.x);
#pragma unroll
        for (int b = 0; b < BATCH; b++) {
            const uint32_t *xb = xg + (size_t)b * (a.cols / 2) + (size_t)c.cb * 128;
            const uint32_t v0 = xb[c.lane], v1 = xb[c.lane + 64];
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
        LaneDec d;
        const bool ok = lw_lane_init(d, lds, slots, c.l, a);
        constexpr int NG = SPL / 4;           // groups of four symbols per lane
        constexpr int HALF = NG / 2;          // groups per tile row
        if (ok) {
            // activations of one group: Q4 four pairs, Q6 two pairs (four columns) per batch row
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            struct XA {
                u32x4 v[BATCH];
            };
            auto fetch = [&](int g) {
                XA r;
#pragma unroll
                for (int b = 0; b < BATCH; b++) {
                    if constexpr (KIND == LW_Q4_PAIR) {
                        const uint32_t ad = xs_addr + (uint32_t)(b * 512 + 16 * g);
                        r.v[b] = *(__attribute__((address_space(3))) const u32x4 *)(size_t)ad;
                    } else {
                        const uint32_t ad = xs_addr + (uint32_t)(b * 512 + 8 * g);
                        const u32x2 t = *(__attribute__((address_space(3))) const u32x2 *)(size_t)ad;
                        r.v[b] = u32x4{t.x, t.y, 0u, 0u};
                    }
                }
                return r;
            };
            // one call per tile row (p): the accumulator row is a compile-time index
            auto run_row = [&](auto pc) {
                constexpr int p = decltype(pc)::value;
                auto use = [&](int, int j, uint32_t pay, const XA &x) {
#pragma unroll
                    for (int b = 0; b < BATCH; b++) {
                        uint32_t xp;
                        if constexpr (KIND == LW_Q4_PAIR)
                            xp = j == 0 ? x.v[b].x : j == 1 ? x.v[b].y : j == 2 ? x.v[b].z : x.v[b].w;
                        else
                            xp = j < 2 ? x.v[b].x : x.v[b].y;
                        acc[p][b] = lw_dot2(pay, xp, acc[p][b]);
                    }
                };
                if constexpr (KIND == LW_Q4_PAIR)
                    lw_decode_pipelined<N8, N16, HALF, XA>(d, a, [](int) { return 0u; }, fetch, use);
                else
                    lw_decode_pipelined<N8, N16, HALF, XA>(
                        d, a, [](int j) { return (j & 1) ? (LW_TPAY_HI - LW_TPAY) : 0u; }, fetch, use);
            };
            run_row(std::integral_constant<int, 0>{});
            run_row(std::integral_constant<int, 1>{});
        }
        if (!ok)                           // unusable LDS base: poison the output
#pragma unroll
            for (int p = 0; p < 2; p++)
#pragma unroll
                for (int b = 0; b < BATCH; b++) acc[p][b] = __builtin_nanf("");
    }

    // dequantise: y_row = d * sum(q x) - m * sum(x) for this tile row
    float val[2][BATCH];
    if (c.wave_active) {
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const uint32_t w = p ? dm.y : dm.x;
            const float dd = lw_half_lo(w), mm = lw_half_hi(w);
#pragma unroll
            for (int b = 0; b < BATCH; b++) val[p][b] = dd * acc[p][b] - mm * sx[b];
        }
    }
    __syncthreads();                      // tiles no longer read: reuse for the reduction
    float *red = reinterpret_cast<float *>(lds + L.tiles);
    // red[wave][b][row], row = half*64 + 2l + p within the workgroup's 128 rows
#pragma unroll
    for (int p = 0; p < 2; p++)
#pragma unroll
        for (int b = 0; b < BATCH; b++)
            red[(c.wave * BATCH + b) * 128 + c.half * 64 + 2 * c.l + p] = c.lane_active ? val[p][b] : 0.f;
    __syncthreads();

    const int64_t row0 = (int64_t)c.rbp * 128;
    uint32_t *last_flag = reinterpret_cast<uint32_t *>(lds + L.flag);
    lw_finish_rows<BATCH>(a, red, row0, c.g, c.rbp, WAVES, last_flag);
}


// Decode only: restore the fixed-width codes (Q4 packed nibbles, Q6 bytes).
template <int KIND, int N8, int N16>
__global__ __launch_bounds__(256) void k_decode_q(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int SPL = KIND == LW_Q4_PAIR ? 256 : 512;
    const LdsLayout L = lds_layout(1, a.max_words, true);
    const LaneCtx c = lane_ctx(a);
    const int S = a.max_words + 3;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + (c.wave * 2 + c.half) * S * 32;
    lw_stage_tab(lds, a.tab, a.min_len, a.max_len, true);
    if (c.wave_active) {
        const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
        lw_stage_tile(slots, a.words, w0, (w1 - w0) >> 5, c.l);
    }
    __syncthreads();
    if (!c.wave_active) return;
    LaneDec d;
    if (!lw_lane_init(d, lds, slots, c.l, a)) return;
    uint32_t *out = reinterpret_cast<uint32_t *>(a.out);
    const int64_t row_bytes = KIND == LW_Q4_PAIR ? a.cols / 2 : a.cols;
    constexpr int NG = SPL / 4;
    constexpr int HALF = NG / 2;
    uint32_t *orow0 = out + (((int64_t)c.rb * 64 + 2 * c.l) * row_bytes + (int64_t)c.cb * (SPL / 2)) / 4;
    uint32_t *orow1 = orow0 + row_bytes / 4;
    struct NoAux {};
    uint32_t pk = 0;
    auto run_row = [&](uint32_t *orow) {
        lw_decode_pipelined<N8, N16, HALF, NoAux>(
            d, a, [](int) { return LW_TPAY_HI - LW_TPAY; }, [](int) { return NoAux{}; },
            [&](int g, int j, uint32_t sym, const NoAux &) {
                pk |= sym << (8 * j);
                if (j == 3) {
                    if (c.lane_active) orow[g] = pk;
                    pk = 0;
                }
            });
    };
    run_row(orow0);
    run_row(orow1);
    if (a.lane_bits && c.lane_active) a.lane_bits[(size_t)c.t * 32 + c.l] = d.u - 31;
}

template <int KIND, int N8, int N16, int BATCH>
hipError_t launch_gemv_q(const KArgs &a, hipStream_t s)
{
    const LdsLayout L = lds_layout(BATCH, a.max_words, false);
    dim3 grid((unsigned)a.groups, (unsigned)((a.n_rb + 1) / 2));
    auto kern = k_gemv_q<KIND, N8, N16, BATCH>;
    hipError_t e = lw_allow_lds<k_gemv_q<KIND, N8, N16, BATCH>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(256), L.total, s, a);
    return hipGetLastError();
}

template <int KIND, int N8, int N16>
hipError_t launch_decode_q(const KArgs &a, hipStream_t s)
{
    const LdsLayout L = lds_layout(1, a.max_words, true);
    dim3 grid((unsigned)a.groups, (unsigned)((a.n_rb + 1) / 2));
    auto kern = k_decode_q<KIND, N8, N16>;
    hipError_t e = lw_allow_lds<k_decode_q<KIND, N8, N16>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(256), L.total, s, a);
    return hipGetLastError();
}

template <int KIND, int N8, int N16>
hipError_t gemv_batch(const KArgs &a, int batch, hipStream_t s)
{
    switch (batch) {
    case 1: return launch_gemv_q<KIND, N8, N16, 1>(a, s);
    case 2: return launch_gemv_q<KIND, N8, N16, 2>(a, s);
    case 3: return launch_gemv_q<KIND, N8, N16, 3>(a, s);
    case 4: return launch_gemv_q<KIND, N8, N16, 4>(a, s);
    case 5: return launch_gemv_q<KIND, N8, N16, 5>(a, s);
    case 6: return launch_gemv_q<KIND, N8, N16, 6>(a, s);
    case 7: return launch_gemv_q<KIND, N8, N16, 7>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int KIND>
hipError_t gemv_plan(const KArgs &a, SadPlan p, int batch, hipStream_t s)
{
    const int code = p.n8ops * 2 + p.n16ops;
    switch (code) {
    case 0: return gemv_batch<KIND, 0, 0>(a, batch, s);
    case 1: return gemv_batch<KIND, 0, 1>(a, batch, s);
    case 2: return gemv_batch<KIND, 1, 0>(a, batch, s);
    case 3: return gemv_batch<KIND, 1, 1>(a, batch, s);
    case 4: return gemv_batch<KIND, 2, 0>(a, batch, s);
    case 5: return gemv_batch<KIND, 2, 1>(a, batch, s);
    }
    return hipErrorInvalidValue;
}

template <int KIND>
hipError_t decode_plan(const KArgs &a, SadPlan p, hipStream_t s)
{
    const int code = p.n8ops * 2 + p.n16ops;
    switch (code) {
    case 0: return launch_decode_q<KIND, 0, 0>(a, s);
    case 1: return launch_decode_q<KIND, 0, 1>(a, s);
    case 2: return launch_decode_q<KIND, 1, 0>(a, s);
    case 3: return launch_decode_q<KIND, 1, 1>(a, s);
    case 4: return launch_decode_q<KIND, 2, 0>(a, s);
    case 5: return launch_decode_q<KIND, 2, 1>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t lw_lds_bytes(int kind, int batch, int max_words, bool decode_only)
{
    (void)kind;
    return lds_layout(batch, max_words, decode_only).total;
}

hipError_t lw_launch_gemv_q(const KArgs &a, int kind, SadPlan p, int batch, hipStream_t s)
{
    if (kind == LW_Q4_PAIR) return gemv_plan<LW_Q4_PAIR>(a, p, batch, s);
    if (kind == LW_Q6_SINGLE) return gemv_plan<LW_Q6_SINGLE>(a, p, batch, s);
    return hipErrorInvalidValue;
}

hipError_t lw_launch_decode_q(const KArgs &a, int kind, SadPlan p, hipStream_t s)
{
    if (kind == LW_Q4_PAIR) return decode_plan<LW_Q4_PAIR>(a, p, s);
    if (kind == LW_Q6_SINGLE) return decode_plan<LW_Q6_SINGLE>(a, p, s);
    return hipErrorInvalidValue;
}
