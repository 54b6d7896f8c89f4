// fused_q.hip -- fused decode + dequantise + GEMV (batch 1..7, VALU) and
// decode-only kernels for 4-bit pair and 6-bit single codes, gfx950.
//
// Work split ("LazyWeights", section "2 . Code them": a 64x256 tile is 32
// lanes of two rows; Fig. 3 caption: recorded offsets let a decoder start
// without the rest).  The bundle records where each of P parts of a tile row
// starts in its lane stream (P = 1, 2, 4 or 8, chosen when the bundle is
// built), and one wavefront decodes one part of a tile: lane l < 32 decodes
// lane stream l's part in tile row 2l, lane l + 32 the same part of row
// 2l+1.  So every lane runs one serial chain of 128/P (Q4) or 256/P (Q6)
// symbols, and all 64 lanes consume the same activation pair at each step
// (x is read once per wavefront from LDS).  The parts of one tile share its
// staged words.  More parts shorten the chains of small matrices and spread
// a large one evenly over the SIMDs (3584 tiles in two parts are seven
// wavefronts on every SIMD of 256 CUs, where whole rows leave some SIMDs four
// and others three or none).
// A workgroup holds whole column blocks of one row band: in parts, eight
// wavefronts (four tiles in two parts, two in four, one in eight); in whole
// rows, sixteen (a whole row band of 13 to 16 column blocks, when there are
// enough row bands to fill the chip), fourteen or four.  The column groups
// of a row band meet in the exchange tree of lane_decode.hpp, so the result
// is deterministic.  When the whole grid is resident at once, each wavefront
// lowers its issue priority as its decode progresses, so the wavefronts
// sharing a SIMD finish together.
//
// Dequantisation w = d*q - m per 256-weight super-block (one tile row) is
// applied after the dot product: y = d * sum(q x) - m * sum(x).
#include <type_traits>

#include "lane_decode.hpp"

namespace {

constexpr int WAVES = 4;                 // wavefronts per workgroup (one column block each), by default

struct LdsLayout {
    uint32_t x, tiles, total;
};

// staged tiles: one per `parts` wavefronts
__host__ __device__ inline LdsLayout lds_layout(int batch, int max_words, bool decode_only, int waves = WAVES,
                                                int parts = 1)
{
    LdsLayout L;
    L.x = LW_TAB_BYTES;
    const uint32_t xbytes = decode_only ? 0u : (uint32_t)(waves * batch * 128 * 4);
    L.tiles = L.x + xbytes;
    const uint32_t tiles = (uint32_t)((waves / parts) * (max_words + 3) * 128);
    const uint32_t red = (uint32_t)(waves * batch * 64 * 4);
    L.total = L.tiles + (tiles > red ? tiles : red);
    return L;
}

// Identity of a lane within the grid: wavefront w of a workgroup decodes
// part p = w % parts of the tile in its slot ts = w / parts.
struct LaneCtx {
    int wave, lane, half, l, g, cb, rb, t, ts, p;
    bool active;
};

LW_DEV LaneCtx lane_ctx(const KArgs &a, int waves = WAVES, int parts = 1)
{
    LaneCtx c;
    c.wave = (int)lw_wave_id();
    c.lane = threadIdx.x & 63;
    c.half = c.lane >> 5;                 // tile row parity decoded by this lane
    c.l = c.lane & 31;                    // lane stream of the tile
    c.g = blockIdx.x;
    c.rb = blockIdx.y;
    c.ts = c.wave / parts;
    c.p = c.wave % parts;
    c.cb = c.g * (waves / parts) + c.ts;
    c.active = c.cb < a.n_cb;
    c.t = c.rb * a.n_cb + (c.active ? c.cb : 0);
    return c;
}

// WPG wavefronts per workgroup decode P parts of WPG/P consecutive column
// blocks of one row band; when they cover whole rows the reduction stays in
// LDS.
template <int KIND, int PLAN, int BATCH, int WPG, int P>
__global__ __launch_bounds__(64 * WPG) void k_gemv_q(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    static_assert(WPG % P == 0, "whole tiles per workgroup");
    constexpr int SPL = KIND == LW_Q4_PAIR ? 256 : 512;
    constexpr int NG = SPL / 8 / P;       // groups of four symbols per part of a tile row
    const LdsLayout L = lds_layout(BATCH, a.max_words, false, WPG, P);
    const LaneCtx c = lane_ctx(a, WPG, P);
    const int S = a.max_words + 3;
    const uint32_t xs_addr = (uint32_t)(size_t)(lds + L.x) + 4u * (uint32_t)(c.wave * BATCH * 128);
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + c.ts * S * 32;

    // Issue every global load first (unconditionally: an inactive wavefront
    // reads tile 0 and drops it), tile offsets first since the tile words
    // depend on them.  Only the decoder table is shared by the workgroup, so
    // the barrier waits for the table stores alone; each wavefront then
    // stores its own tile and activations and starts decoding as soon as its
    // own data is in (a wavefront's LDS operations complete in order).
    const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
    const LwTabRegs tr = lw_tab_fetch<PLAN>(a, false);
    const uint32_t dm = a.dm[(size_t)c.t * 64 + 2 * c.l + c.half];   // (d, m) of this lane's tile row
    // this lane's part: bundle part half * parts + p * (parts / P)
    const uint32_t start = lw_part_start(a, c.t, c.l, c.half * a.parts + c.p * (a.parts / P));
    uint32_t xv[BATCH][2];
    const uint32_t *xg = reinterpret_cast<const uint32_t *>(a.x) + (size_t)(c.active ? c.cb : 0) * 128;
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
        xv[b][0] = xg[(size_t)b * (a.cols / 2) + c.lane];
        xv[b][1] = xg[(size_t)b * (a.cols / 2) + c.lane + 64];
    }
    // With 14 or 16 wavefronts a workgroup (one workgroup a CU) the tile
    // loads go out after the table barrier instead: issued before it, a
    // wavefront whose loads the memory system holds back (the whole matrix
    // is requested at once) reaches the barrier late and stalls all of
    // them, about 5 % on a 16-block row band; with four wavefronts the
    // order makes no difference.
    // In parts, the tile's first wavefront stages it for all of them, and
    // one barrier then covers the table and the tiles.
    LwTileRegs64 tile;
    if constexpr (P > 1) {
        if (c.p == 0) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        lw_tab_put<PLAN>(lds, tr, a);
        if (c.p == 0) lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    } else {
        if constexpr (WPG <= WAVES) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        lw_tab_put<PLAN>(lds, tr, a);
        __syncthreads();                  // the decoder table is complete
        if constexpr (WPG > WAVES) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    }
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
        *(lw_lds_w32 *)(size_t)(xs_addr + 4u * (b * 128 + c.lane)) = xv[b][0];
        *(lw_lds_w32 *)(size_t)(xs_addr + 4u * (b * 128 + c.lane + 64)) = xv[b][1];
    }
    if constexpr (P > 1)
        __syncthreads();                  // the table and every tile of the workgroup are complete
    else
        lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);

    float acc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; b++) acc[b] = 0.f;

    if (c.active) {
        LaneDec d;
        const bool ok = lw_lane_init(d, lds, slots, c.l, a);
        d.advance(start);
        const int g0 = c.p * NG;          // first group of this part within the tile row
        if (ok) {
            // activations of one group: Q4 four pairs, Q6 two pairs (four columns) per batch row
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            struct XA {
                u32x4 v[BATCH];
            };
            auto fetch = [&](int g) {
                lw_ramp<NG>(a.ramp, g);
                XA r;
#pragma unroll
                for (int b = 0; b < BATCH; b++) {
                    if constexpr (KIND == LW_Q4_PAIR) {
                        const uint32_t ad = xs_addr + (uint32_t)(b * 512 + 16 * (g0 + g));
                        r.v[b] = *(__attribute__((address_space(3))) const u32x4 *)(size_t)ad;
                    } else {
                        const uint32_t ad = xs_addr + (uint32_t)(b * 512 + 8 * (g0 + g));
                        const u32x2 t = *(__attribute__((address_space(3))) const u32x2 *)(size_t)ad;
                        r.v[b] = u32x4{t.x, t.y, 0u, 0u};
                    }
                }
                return r;
            };
            auto use = [&](int, int j, uint32_t pay, const XA &x) {
#pragma unroll
                for (int b = 0; b < BATCH; b++) {
                    uint32_t xp;
                    if constexpr (KIND == LW_Q4_PAIR)
                        xp = j == 0 ? x.v[b].x : j == 1 ? x.v[b].y : j == 2 ? x.v[b].z : x.v[b].w;
                    else
                        xp = j < 2 ? x.v[b].x : x.v[b].y;
                    acc[b] = lw_dot2(pay, xp, acc[b]);
                }
            };
            if constexpr (KIND == LW_Q4_PAIR)
                lw_decode_pipelined<PLAN, NG, XA, true>(d, a, [](int) { return 0u; }, fetch, use);
            else
                lw_decode_pipelined<PLAN, NG, XA, true>(
                    d, a, [](int j) { return (j & 1) ? (LW_TPAY_HI - LW_TPAY) : 0u; }, fetch, use);
        } else {                           // unusable LDS base: poison the output
#pragma unroll
            for (int b = 0; b < BATCH; b++) acc[b] = __builtin_nanf("");
        }
    }

    // dequantise: y_row = d * sum(q x) - m * sum(x) over this part's columns
    // of the tile row (the activation sum is taken here, off the decode's
    // start; lane i holds the column pairs i and i + 64)
    const bool in0 = c.lane / (128 / P) == c.p, in1 = (c.lane + 64) / (128 / P) == c.p;
    float sx[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; b++)
        sx[b] = lw_wave_sum((in0 ? lw_half_lo(xv[b][0]) + lw_half_hi(xv[b][0]) : 0.f) +
                            (in1 ? lw_half_lo(xv[b][1]) + lw_half_hi(xv[b][1]) : 0.f));
    float val[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; b++) val[b] = c.active ? lw_half_lo(dm) * acc[b] - lw_half_hi(dm) * sx[b] : 0.f;
    __syncthreads();                      // tiles no longer read: reuse for the reduction
    float *red = reinterpret_cast<float *>(lds + L.tiles);
    // red[wave][b][row], row = 2l + half within the tile's 64 rows
#pragma unroll
    for (int b = 0; b < BATCH; b++) red[(c.wave * BATCH + b) * 64 + 2 * c.l + c.half] = val[b];
    __syncthreads();

    lw_finish_rows<BATCH, 64>(a, red, (int64_t)c.rb * 64, c.g, WPG);
}


// Balanced layout (bundles in parts, batch 1..4).  With U = 4K + 2 tiles per
// CU (14336x4096 and 4096x14336 on 256 CUs: 3584 tiles, U = 14), whole
// tiles give some SIMDs K + 1 tiles of work and others K.  Here one
// workgroup per CU takes U consecutive tiles in row-major order with 4K + 4
// wavefronts: wavefronts 0 .. 4K-1 decode tiles 0 .. 4K-1 whole, and
// wavefronts 4K .. 4K+3 decode the two halves (recorded parts) of tiles 4K
// and 4K+1.  A workgroup's wavefronts w, w+4, w+8, ... share a SIMD, so every
// SIMD gets K + 1/2 tiles.  Every wavefront stages its tile in its own slot
// after the table barrier, as in the whole-row layout, so it starts decoding
// when its own tile is in (one shared staging would need a barrier after the
// slowest tile of the workgroup); the second request of a split tile's lines
// is served by the CU's L2.  A workgroup's tiles span at most two row bands
// (U <= the column blocks); each row band's sums meet those of the other
// workgroups holding its tiles in the exchange tree (leaf = workgroup - the
// band's first workgroup).
__host__ __device__ inline LdsLayout lds_layout_bal(int batch, int max_words, int waves, int tiles_per_wg)
{
    LdsLayout L;
    L.x = LW_TAB_BYTES;
    L.tiles = L.x + (uint32_t)(waves * batch * 128 * 4);
    const uint32_t tiles = (uint32_t)(tiles_per_wg * (max_words + 3) * 128);
    const uint32_t red = (uint32_t)(waves * batch * 64 * 4);
    L.total = L.tiles + (tiles > red ? tiles : red);
    return L;
}

template <int KIND, int PLAN, int BATCH, int K>
__global__ __launch_bounds__(64 * (4 * K + 4)) void k_gemv_bal(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int WPG = 4 * K + 4, U = 4 * K + 2;   // wavefronts and tiles of a workgroup
    constexpr int SPL = KIND == LW_Q4_PAIR ? 256 : 512;
    constexpr int NG = SPL / 8;           // groups of four symbols per tile row (half tiles: NG / 2)
    const LdsLayout L = lds_layout_bal(BATCH, a.max_words, WPG, WPG);
    const int wave = (int)lw_wave_id(), lane = threadIdx.x & 63, half = lane >> 5, l = lane & 31;
    const bool split = wave >= 4 * K;     // a half-tile wavefront
    const int j = split ? 4 * K + ((wave - 4 * K) >> 1) : wave;   // tile slot within the workgroup
    const int p = split ? ((wave - 4 * K) & 1) : 0;                  // half of the tile row
    const int64_t T0 = (int64_t)blockIdx.x * U;                      // the workgroup's first tile
    const int64_t t = T0 + j;             // tiles are in row-major order: t = rb * n_cb + cb
    const int cb = (int)(t % a.n_cb);
    const int S = a.max_words + 3;
    const uint32_t xs_addr = (uint32_t)(size_t)(lds + L.x) + 4u * (uint32_t)(wave * BATCH * 128);
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + wave * S * 32;

    // Issue every global load first (as in k_gemv_q); the tile loads go out
    // after the table barrier, as in the sixteen-wavefront whole-row layout.
    const uint32_t w0 = a.tile_off[t], w1 = a.tile_off[t + 1];
    const LwTabRegs tr = lw_tab_fetch<PLAN>(a, false);
    const uint32_t dm = a.dm[(size_t)t * 64 + 2 * l + half];
    const uint32_t start = lw_part_start(a, t, l, half * a.parts + p * (a.parts / 2));
    uint32_t xv[BATCH][2];
    const uint32_t *xg = reinterpret_cast<const uint32_t *>(a.x) + (size_t)cb * 128;
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
        xv[b][0] = xg[(size_t)b * (a.cols / 2) + lane];
        xv[b][1] = xg[(size_t)b * (a.cols / 2) + lane + 64];
    }
    lw_tab_put<PLAN>(lds, tr, a);
    __syncthreads();                      // the decoder table is complete
    LwTileRegs64 tile;
    lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, lane, tile);
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
        *(lw_lds_w32 *)(size_t)(xs_addr + 4u * (b * 128 + lane)) = xv[b][0];
        *(lw_lds_w32 *)(size_t)(xs_addr + 4u * (b * 128 + lane + 64)) = xv[b][1];
    }
    lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, lane, tile);

    float acc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; b++) acc[b] = 0.f;
    {
        LaneDec d;
        const bool ok = lw_lane_init(d, lds, slots, l, a);
        d.advance(start);
        const int g0 = p * (NG / 2);      // first group of this wavefront's columns
        if (ok) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            struct XA {
                u32x4 v[BATCH];
            };
            auto fetch_x = [&](int g) {
                XA r;
#pragma unroll
                for (int b = 0; b < BATCH; b++) {
                    if constexpr (KIND == LW_Q4_PAIR) {
                        const uint32_t ad = xs_addr + (uint32_t)(b * 512 + 16 * (g0 + g));
                        r.v[b] = *(__attribute__((address_space(3))) const u32x4 *)(size_t)ad;
                    } else {
                        const uint32_t ad = xs_addr + (uint32_t)(b * 512 + 8 * (g0 + g));
                        const u32x2 t2 = *(__attribute__((address_space(3))) const u32x2 *)(size_t)ad;
                        r.v[b] = u32x4{t2.x, t2.y, 0u, 0u};
                    }
                }
                return r;
            };
            auto use = [&](int, int jj, uint32_t pay, const XA &x) {
#pragma unroll
                for (int b = 0; b < BATCH; b++) {
                    uint32_t xp;
                    if constexpr (KIND == LW_Q4_PAIR)
                        xp = jj == 0 ? x.v[b].x : jj == 1 ? x.v[b].y : jj == 2 ? x.v[b].z : x.v[b].w;
                    else
                        xp = jj < 2 ? x.v[b].x : x.v[b].y;
                    acc[b] = lw_dot2(pay, xp, acc[b]);
                }
            };
            auto pay_off = [](int jj) { return (KIND != LW_Q4_PAIR && (jj & 1)) ? (LW_TPAY_HI - LW_TPAY) : 0u; };
            if (split)
                lw_decode_pipelined<PLAN, NG / 2, XA, true>(
                    d, a, pay_off, [&](int g) { lw_ramp<NG / 2>(a.ramp, g); return fetch_x(g); }, use);
            else
                lw_decode_pipelined<PLAN, NG, XA, true>(
                    d, a, pay_off, [&](int g) { lw_ramp<NG>(a.ramp, g); return fetch_x(g); }, use);
        } else {                           // unusable LDS base: poison the output
#pragma unroll
            for (int b = 0; b < BATCH; b++) acc[b] = __builtin_nanf("");
        }
    }

    // dequantise over this wavefront's columns (lane i holds the column pairs i and i + 64)
    const bool in0 = !split || p == 0, in1 = !split || p == 1;
    float sx[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; b++)
        sx[b] = lw_wave_sum((in0 ? lw_half_lo(xv[b][0]) + lw_half_hi(xv[b][0]) : 0.f) +
                            (in1 ? lw_half_lo(xv[b][1]) + lw_half_hi(xv[b][1]) : 0.f));
    __syncthreads();                      // tiles no longer read: reuse for the partial sums
    float *red = reinterpret_cast<float *>(lds + L.tiles);
#pragma unroll
    for (int b = 0; b < BATCH; b++)
        red[(wave * BATCH + b) * 64 + 2 * l + half] = lw_half_lo(dm) * acc[b] - lw_half_hi(dm) * sx[b];
    __syncthreads();

    lw_finish_balanced<BATCH, 64, K>(a, red);
}

// Decode only: restore the fixed-width codes (Q4 packed nibbles, Q6 bytes).
template <int KIND, int PLAN>
__global__ __launch_bounds__(256) void k_decode_q(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int SPL = KIND == LW_Q4_PAIR ? 256 : 512;
    const LdsLayout L = lds_layout(1, a.max_words, true);
    const LaneCtx c = lane_ctx(a);
    const int S = a.max_words + 3;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + c.wave * S * 32;
    // issue, then store (as in k_gemv_q)
    const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
    const LwTabRegs tr = lw_tab_fetch<PLAN>(a, true);
    const uint32_t start = lw_part_start(a, c.t, c.l, c.half * a.parts);   // this lane's tile row
    LwTileRegs64 tile;
    lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    lw_tab_put<PLAN>(lds, tr, a);
    __syncthreads();
    if (!c.active) return;
    lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    LaneDec d;
    if (!lw_lane_init(d, lds, slots, c.l, a)) return;
    d.advance(start);
    const int64_t row_bytes = KIND == LW_Q4_PAIR ? a.cols / 2 : a.cols;
    constexpr int NG = SPL / 8;           // groups of four symbols per tile row
    // The lane's restored row segment (4 bytes per group) is collected in
    // registers and leaves as 16-byte stores that fill whole 128-byte lines
    // (the loops are unrolled, so every index is a compile-time constant).
    // 4-bit rows store every four groups, from inside the decode loop, so the
    // writes overlap decoding (14336x4096: 22.4 against 23.6 us when each
    // row left in one burst); 6-bit rows, with twice the output per coded
    // bit, keep one burst of whole lines per 32 groups (16-byte pieces spread
    // over the decode measured 13 % slower on 28672x8192).  Rows decode 32
    // groups at a time (one unrolled run of all 64 6-bit groups measured
    // 17 % slower).
    uint4 *orow = reinterpret_cast<uint4 *>(static_cast<uint8_t *>(a.out) +
                                            ((int64_t)c.rb * 64 + 2 * c.l + c.half) * row_bytes +
                                            (int64_t)c.cb * (SPL / 2));
    constexpr int RUN = 32;
    constexpr int SG = KIND == LW_Q4_PAIR ? 4 : RUN;   // groups per batch of stores
    struct NoAux {};
    uint32_t buf[SG];
    uint32_t pk = 0;
#pragma unroll
    for (int r = 0; r < NG / RUN; r++) {
        lw_decode_pipelined<PLAN, RUN, NoAux, true>(
            d, a, [](int) { return LW_TPAY_HI - LW_TPAY; },
            [](int) { return NoAux{}; },
            [&](int g, int j, uint32_t sym, const NoAux &) {
                pk |= sym << (8 * j);
                if (j == 3) {
                    buf[g % SG] = pk;
                    pk = 0;
                    if (g % SG == SG - 1) {
                        const int o = r * (RUN / 4) + (g - (SG - 1)) / 4;   // first 16-byte word of the batch
#pragma unroll
                        for (int i = 0; i < SG / 4; i++)
                            orow[o + i] = make_uint4(buf[4 * i], buf[4 * i + 1], buf[4 * i + 2], buf[4 * i + 3]);
                    }
                }
            });
    }
    // the lane of the second row ends where the whole lane stream ends
    if (a.lane_bits && c.half) a.lane_bits[(size_t)c.t * 32 + c.l] = d.bitpos();
}

template <int KIND, int PLAN, int BATCH, int WPG, int P = 1>
hipError_t launch_gemv_wpg(const KArgs &a0, hipStream_t s)
{
    KArgs a = a0;
    constexpr int TPW = WPG / P;          // column blocks per workgroup
    a.groups = (a.n_cb + TPW - 1) / TPW;  // column groups combined through the workspace (none if 1)
    if (a.groups > 1 && a.groups > lw_work_groups(a.n_cb, a.parts)) return hipErrorInvalidValue;
    a.ramp = lw_resident_ramp((int64_t)a.n_rb * a.n_cb * P);
    const LdsLayout L = lds_layout(BATCH, a.max_words, false, WPG, P);
    dim3 grid((unsigned)a.groups, (unsigned)a.n_rb);
    auto kern = k_gemv_q<KIND, PLAN, BATCH, WPG, P>;
    hipError_t e = lw_allow_lds<k_gemv_q<KIND, PLAN, BATCH, WPG, P>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(64 * WPG), L.total, s, a);
    return hipGetLastError();
}

template <int KIND, int PLAN, int BATCH, int K>
hipError_t launch_gemv_bal(const KArgs &a0, hipStream_t s)
{
    KArgs a = a0;
    constexpr int WPG = 4 * K + 4;
    a.ramp = 1;                           // one workgroup per CU: the whole grid is resident
    const LdsLayout L = lds_layout_bal(BATCH, a.max_words, WPG, WPG);
    auto kern = k_gemv_bal<KIND, PLAN, BATCH, K>;
    hipError_t e = lw_allow_lds<k_gemv_bal<KIND, PLAN, BATCH, K>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)a.n_rb * a.n_cb / (4 * K + 2))), dim3(64 * WPG), L.total, s, a);
    return hipGetLastError();
}

// The balanced layout applies when the tiles are U = 4K + 2 per CU (K = 1..3),
// the bundle records half-row starts (parts >= 2), a workgroup's tiles span
// at most two row bands, the staged tiles fit in LDS and the workspace holds
// the widest band's tree.  Returns hipErrorNotSupported otherwise.
template <int KIND, int PLAN, int BATCH>
hipError_t try_gemv_bal(const KArgs &a, hipStream_t s)
{
    const int cus = lw_device_cu_count();
    const int64_t tiles = (int64_t)a.n_rb * a.n_cb;
    if (cus <= 0 || a.parts < 2 || tiles % cus) return hipErrorNotSupported;
    const int64_t U = tiles / cus;
    if (U % 4 != 2 || U < 6 || U > 14 || a.n_cb < U) return hipErrorNotSupported;
    if (lds_layout_bal(BATCH, a.max_words, (int)U + 2, (int)U + 2).total > (uint32_t)lw_device_lds_bytes())
        return hipErrorNotSupported;
    if ((a.n_cb + U - 1) / U + 1 > lw_work_groups(a.n_cb, a.parts)) return hipErrorNotSupported;
    if (U == 6) return launch_gemv_bal<KIND, PLAN, BATCH, 1>(a, s);
    if (U == 10) return launch_gemv_bal<KIND, PLAN, BATCH, 2>(a, s);
    return launch_gemv_bal<KIND, PLAN, BATCH, 3>(a, s);
}

// At batch 1..4 the balanced layout goes first where it applies (bundles in
// parts with 4K + 2 tiles per CU; 4096x14336: 19.2 against 20.4-20.8 us in
// fourteen-wavefront groups).  Bundles in parts for their size (up to 2048
// tiles) decode every recorded part in eight-wavefront workgroups (measured
// best at 16 to 2048 tiles); other bundles are decoded in whole rows.  In whole
// rows: 16 wavefronts, no cross-workgroup reduction, when a row band has
// 13..16 column blocks, the tiles fit in LDS and there are at least 128 row
// bands (fewer leave most CUs idle: 1024x4096 takes 16.1 us so, 9.9 us in
// four-wavefront groups); 14 wavefronts (a few column groups, every
// wavefront active) when the column blocks are a multiple of 14 (K = 14336
// and 28672; plans of at most eight comparisons) and the whole grid is
// resident at once (with several generations, workgroups this large free
// their CU only all together: 8 % slower on 8192x28672); else four.
template <int KIND, int PLAN, int BATCH>
hipError_t launch_gemv_q(const KArgs &a, hipStream_t s)
{
    const uint32_t lds = (uint32_t)lw_device_lds_bytes();
    if constexpr (BATCH <= 4) {
        const hipError_t e = try_gemv_bal<KIND, PLAN, BATCH>(a, s);
        if (e != hipErrorNotSupported) return e;
    }
    // the eight-wavefront part layouts serve the bundles the part rule puts
    // in parts for their size (tiles x parts within LW_PART_UNITS)
    const bool small = (int64_t)a.n_rb * a.n_cb * a.parts <= LW_PART_UNITS;
    if (small && a.parts == 2 && lds_layout(BATCH, a.max_words, false, 8, 2).total <= lds)
        return launch_gemv_wpg<KIND, PLAN, BATCH, 8, 2>(a, s);
    if (small && a.parts == 4 && lds_layout(BATCH, a.max_words, false, 8, 4).total <= lds)
        return launch_gemv_wpg<KIND, PLAN, BATCH, 8, 4>(a, s);
    if (small && a.parts == 8 && lds_layout(BATCH, a.max_words, false, 8, 8).total <= lds)
        return launch_gemv_wpg<KIND, PLAN, BATCH, 8, 8>(a, s);
    if constexpr (BATCH <= 4) {
        if (a.n_cb > 12 && a.n_cb <= 16 && a.n_rb >= 128 && lds_layout(BATCH, a.max_words, false, 16).total <= lds)
            return launch_gemv_wpg<KIND, PLAN, BATCH, 16>(a, s);
        if constexpr (PLAN != LW_P_GEN) {
            if (a.n_cb > 16 && a.n_cb % 14 == 0 && lw_resident_ramp((int64_t)a.n_rb * a.n_cb) &&
                lds_layout(BATCH, a.max_words, false, 14).total <= lds)
                return launch_gemv_wpg<KIND, PLAN, BATCH, 14>(a, s);
        }
    }
    return launch_gemv_wpg<KIND, PLAN, BATCH, WAVES>(a, s);
}

template <int KIND, int PLAN>
hipError_t launch_decode_q(const KArgs &a, hipStream_t s)
{
    const LdsLayout L = lds_layout(1, a.max_words, true);
    dim3 grid((unsigned)((a.n_cb + WAVES - 1) / WAVES), (unsigned)a.n_rb);   // one column block per wavefront
    auto kern = k_decode_q<KIND, PLAN>;
    hipError_t e = lw_allow_lds<k_decode_q<KIND, PLAN>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(256), L.total, s, a);
    return hipGetLastError();
}

template <int KIND, int PLAN>
hipError_t gemv_batch(const KArgs &a, int batch, hipStream_t s)
{
    switch (batch) {
    case 1: return launch_gemv_q<KIND, PLAN, 1>(a, s);
    case 2: return launch_gemv_q<KIND, PLAN, 2>(a, s);
    case 3: return launch_gemv_q<KIND, PLAN, 3>(a, s);
    case 4: return launch_gemv_q<KIND, PLAN, 4>(a, s);
    case 5: return launch_gemv_q<KIND, PLAN, 5>(a, s);
    case 6: return launch_gemv_q<KIND, PLAN, 6>(a, s);
    case 7: return launch_gemv_q<KIND, PLAN, 7>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int KIND>
hipError_t gemv_plan(const KArgs &a, SadPlan p, int batch, hipStream_t s)
{
    return lw_with_plan(p, [&](auto P) { return gemv_batch<KIND, decltype(P)::value>(a, batch, s); });
}

template <int KIND>
hipError_t decode_plan(const KArgs &a, SadPlan p, hipStream_t s)
{
    return lw_with_plan(p, [&](auto P) { return launch_decode_q<KIND, decltype(P)::value>(a, s); });
}

}  // namespace

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
