// bf16.hip -- fused exponent-decode + GEMV (batch 1..7) and decode-only for
// bf16 weights whose exponent byte is Huffman coded ("Unweight: Compressing
// LLM Weights for Faster Inference", sections "Understanding BF16 weight
// structure" and "The exponent's exploitable redundancy"), gfx950.
//
// Palette indices are decoded with the same per-lane decoder and work split
// as the quantised kernels: one wavefront per tile, lane l + 32*half decodes
// the 256 single symbols of tile row 2l + half (the second row from the
// lane's split bit).  Payload
// tables hold the palette exponent pre-shifted to the low (<< 7) and high
// (<< 23) bf16 of a pair.  The raw sign+mantissa bytes of a lane come as one
// 32-bit word per four columns, coalesced across the lanes; every lane uses
// them at the same rate, so they stream into a register ring one 16-group
// chunk ahead of use.  A pair of weights is rebuilt as
//   ((perm of the two sm bytes) & 0x807F807F) | e0 << 7 | e1 << 23
// and consumed by v_dot2c_f32_bf16.  A 64-weight row segment stored verbatim
// (an exponent outside the palette) was coded with the placeholder palette
// index 0; after the main loop the rare lanes that own such segments add
// (verbatim - placeholder weight) * x for its 64 columns.
#include <type_traits>

#include "lane_decode.hpp"

namespace {

constexpr int WAVES = 4;
constexpr int CHUNK = 16;                 // groups of four columns per sm prefetch chunk

struct LdsLayout {
    uint32_t x, tiles, total;
};

__host__ __device__ inline LdsLayout lds_layout(int batch, int max_words, bool decode_only, int waves = WAVES)
{
    LdsLayout L;
    L.x = LW_TAB_BYTES;
    const uint32_t xbytes = decode_only ? 0u : (uint32_t)(waves * batch * 128 * 4);
    L.tiles = L.x + xbytes;
    const uint32_t tiles = (uint32_t)(waves * (max_words + 3) * 128);
    const uint32_t red = (uint32_t)(waves * batch * 64 * 4);
    L.total = L.tiles + (tiles > red ? tiles : red);
    return L;
}

// Identity of a lane: one wavefront per tile, lane l + 32*half decodes tile
// row 2l + half (the second row from the lane's split bit).
struct LaneCtx {
    int wave, lane, half, l, g, cb, rb, t;
    bool active;
};

LW_DEV LaneCtx lane_ctx(const KArgs &a, int waves = WAVES)
{
    LaneCtx c;
    c.wave = (int)lw_wave_id();
    c.lane = threadIdx.x & 63;
    c.half = c.lane >> 5;
    c.l = c.lane & 31;
    c.g = blockIdx.x;
    c.rb = blockIdx.y;
    c.cb = c.g * waves + c.wave;
    c.active = c.cb < a.n_cb;
    c.t = c.rb * a.n_cb + (c.active ? c.cb : 0);
    return c;
}

typedef __bf16 lw_bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

LW_DEV float lw_dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(lw_bf16x2, a), __builtin_bit_cast(lw_bf16x2, b), c,
                                           false);
}

LW_DEV float lw_bf16_to_f32(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

// Two weights (columns j0, j0+1 of a four-column group) from the group's sm
// word and the two decoded exponent payloads.
template <int J0>
LW_DEV uint32_t lw_pair(uint32_t smw, uint32_t pay_lo, uint32_t pay_hi)
{
    const uint32_t spread = __builtin_amdgcn_perm(smw, smw, J0 == 0 ? 0x01010000u : 0x03030202u);
    return (spread & 0x807F807Fu) | pay_lo | pay_hi;
}

// Issue the sm words of one chunk (CHUNK groups) of a lane's row.
LW_DEV void lw_load_sm(uint32_t (&dst)[CHUNK], const uint32_t *smrow, int chunk)
{
#pragma unroll
    for (int i = 0; i < CHUNK; i++) dst[i] = smrow[(chunk * CHUNK + i) * 32];
}

// WPG wavefronts per workgroup, one column block each: four, or sixteen
// (whole rows, the reduction in LDS) as in fused_q.hip.
template <int PLAN, int BATCH, int WPG>
__global__ __launch_bounds__(64 * WPG) void k_gemv_bf16(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const LdsLayout L = lds_layout(BATCH, a.max_words, false, WPG);
    const LaneCtx c = lane_ctx(a, WPG);
    const int S = a.max_words + 3;
    const uint32_t xs_addr = (uint32_t)(size_t)(lds + L.x) + 4u * (uint32_t)(c.wave * BATCH * 128);
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + c.wave * S * 32;
    // the lane's sign+mantissa row: word g holds columns 4g..4g+3
    const uint32_t *smrow = a.sm + (size_t)c.t * 4096 + (size_t)c.half * 64 * 32 + c.l;

    // issue every load, tile offsets first; table barrier; own tile and x (as in fused_q.hip)
    const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
    const LwTabRegs tr = lw_tab_fetch<PLAN>(a, false);
    const uint32_t start = lw_part_start(a, c.t, c.l, c.half * a.parts);   // this lane's tile row
    uint32_t xv[BATCH][2];
    const uint32_t *xg = reinterpret_cast<const uint32_t *>(a.x) + (size_t)(c.active ? c.cb : 0) * 128;
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
        xv[b][0] = xg[(size_t)b * (a.cols / 2) + c.lane];
        xv[b][1] = xg[(size_t)b * (a.cols / 2) + c.lane + 64];
    }
    uint32_t ring[2][CHUNK];
    lw_load_sm(ring[0], smrow, 0);
    // whole-row workgroups request their tiles after the table barrier (see fused_q.hip)
    LwTileRegs64 tile;
    if constexpr (WPG <= WAVES) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    lw_tab_put<PLAN>(lds, tr, a);
    __syncthreads();                      // the decoder table is complete
    if constexpr (WPG > WAVES) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
        *(lw_lds_w32 *)(size_t)(xs_addr + 4u * (b * 128 + c.lane)) = xv[b][0];
        *(lw_lds_w32 *)(size_t)(xs_addr + 4u * (b * 128 + c.lane + 64)) = xv[b][1];
    }
    lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);

    float acc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; b++) acc[b] = 0.f;

    if (c.active) {
        LaneDec d;
        const bool ok = lw_lane_init(d, lds, slots, c.l, a);
        d.advance(start);
        if (ok) {
            struct XA {
                u32x2 v[BATCH];
                uint32_t sm;
            };
            uint32_t pend = 0;
            auto run_chunk = [&](int ch, const uint32_t (&cur)[CHUNK]) {
                auto fetch = [&](int g) {
                    lw_ramp<64>(a.ramp, ch * CHUNK + g);
                    XA r;
#pragma unroll
                    for (int b = 0; b < BATCH; b++) {
                        const uint32_t ad = xs_addr + (uint32_t)(b * 512 + 8 * (ch * CHUNK + g));
                        r.v[b] = *(__attribute__((address_space(3))) const u32x2 *)(size_t)ad;
                    }
                    r.sm = cur[g];
                    return r;
                };
                auto use = [&](int, int j, uint32_t pay, const XA &x) {
                    if (j & 1) {
                        const uint32_t w2 = (j == 1) ? lw_pair<0>(x.sm, pend, pay) : lw_pair<2>(x.sm, pend, pay);
#pragma unroll
                        for (int b = 0; b < BATCH; b++)
                            acc[b] = lw_dot2_bf16(w2, j == 1 ? x.v[b].x : x.v[b].y, acc[b]);
                    } else {
                        pend = pay;
                    }
                };
                lw_decode_pipelined<PLAN, CHUNK, XA, true>(
                    d, a, [](int j) { return (j & 1) ? (LW_TPAY_HI - LW_TPAY) : 0u; }, fetch, use);
            };
#pragma unroll
            for (int ch = 0; ch < 64 / CHUNK; ch += 2) {
                lw_load_sm(ring[1], smrow, ch + 1);
                run_chunk(ch, ring[0]);
                if (ch + 2 < 64 / CHUNK) lw_load_sm(ring[0], smrow, ch + 2);
                run_chunk(ch + 1, ring[1]);
            }

            // verbatim segments (rare): replace the placeholder weights'
            // contribution by the stored values', all lanes on one segment
            const uint16_t *xcol = a.x + (size_t)c.cb * 256;
            lw_verbatim_visit(a, c.t, c.lane, [&](int row, int col, uint32_t vv, uint32_t ph) {
                const float wdiff = lw_bf16_to_f32(vv) - lw_bf16_to_f32(ph);
                const int owner = (row >> 1) + 32 * (row & 1);
#pragma unroll
                for (int b = 0; b < BATCH; b++) {
                    const float sb = lw_wave_sum(wdiff * lw_bf16_to_f32(xcol[(size_t)b * a.cols + col]));
                    if (c.lane == owner) acc[b] += sb;
                }
            });
        } else {
#pragma unroll
            for (int b = 0; b < BATCH; b++) acc[b] = __builtin_nanf("");
        }
    }
    __syncthreads();                      // tiles no longer read: reuse for the reduction
    float *red = reinterpret_cast<float *>(lds + L.tiles);
#pragma unroll
    for (int b = 0; b < BATCH; b++) red[(c.wave * BATCH + b) * 64 + 2 * c.l + c.half] = c.active ? acc[b] : 0.f;
    __syncthreads();
    lw_finish_rows<BATCH, 64>(a, red, (int64_t)c.rb * 64, c.g, WPG);
}

// Decode only: rebuild the bf16 matrix [rows][cols].
template <int PLAN>
__global__ __launch_bounds__(256) void k_decode_bf16(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const LdsLayout L = lds_layout(1, a.max_words, true);
    const LaneCtx c = lane_ctx(a);
    const int S = a.max_words + 3;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + c.wave * S * 32;
    const uint32_t *smrow = a.sm + (size_t)c.t * 4096 + (size_t)c.half * 64 * 32 + c.l;
    const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
    const LwTabRegs tr = lw_tab_fetch<PLAN>(a, false);
    const uint32_t start = lw_part_start(a, c.t, c.l, c.half * a.parts);   // this lane's tile row
    uint32_t ring[2][CHUNK];
    lw_load_sm(ring[0], smrow, 0);
    LwTileRegs64 tile;
    lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    lw_tab_put<PLAN>(lds, tr, a);
    __syncthreads();
    if (!c.active) return;
    lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    LaneDec d;
    if (!lw_lane_init(d, lds, slots, c.l, a)) return;
    d.advance(start);
    // the lane's restored row segment: each chunk of 16 groups (64 weights,
    // 128 bytes) is collected in registers and written as 16-byte stores
    uint4 *orow = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.out) +
                                            ((int64_t)c.rb * 64 + 2 * c.l + c.half) * a.cols + (int64_t)c.cb * 256);
    struct XA {
        uint32_t sm;
    };
    uint32_t pend = 0;
    auto run_chunk = [&](int ch, const uint32_t (&cur)[CHUNK]) {
        uint32_t buf[2 * CHUNK];
        lw_decode_pipelined<PLAN, CHUNK, XA, true>(
            d, a, [](int j) { return (j & 1) ? (LW_TPAY_HI - LW_TPAY) : 0u; },
            [&](int g) { return XA{cur[g]}; },
            [&](int g, int j, uint32_t pay, const XA &x) {
                if (j & 1)
                    buf[2 * g + (j >> 1)] = (j == 1) ? lw_pair<0>(x.sm, pend, pay) : lw_pair<2>(x.sm, pend, pay);
                else
                    pend = pay;
            });
#pragma unroll
        for (int i = 0; i < CHUNK / 2; i++)
            orow[ch * (CHUNK / 2) + i] = make_uint4(buf[4 * i], buf[4 * i + 1], buf[4 * i + 2], buf[4 * i + 3]);
    };
#pragma unroll
    for (int ch = 0; ch < 64 / CHUNK; ch += 2) {
        lw_load_sm(ring[1], smrow, ch + 1);
        run_chunk(ch, ring[0]);
        if (ch + 2 < 64 / CHUNK) lw_load_sm(ring[0], smrow, ch + 2);
        run_chunk(ch + 1, ring[1]);
    }
    // the lane of the second row ends where the whole lane stream ends
    if (a.lane_bits && c.half) a.lane_bits[(size_t)c.t * 32 + c.l] = d.bitpos();
    // verbatim segments overwrite the placeholder weights (rare): after this
    // wavefront's row stores, all lanes write one segment
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint16_t *o16 = reinterpret_cast<uint16_t *>(a.out);
    lw_verbatim_visit(a, c.t, c.lane, [&](int row, int col, uint32_t vv, uint32_t) {
        o16[((int64_t)c.rb * 64 + row) * a.cols + (int64_t)c.cb * 256 + col] = (uint16_t)vv;
    });
}

// Transcode for the reconstructive GEMM ("Unweight", "Four approaches to
// using compressed weights": the runtime palette transcode and the
// exponent-only decode).  The lane decoder runs as in k_decode_bf16 but
// writes, instead of weights, either the 4-bit palette index of every weight
// (EXP = false; eight columns to a 32-bit word, the lowest column in the low
// nibble) or its exponent byte (EXP = true; four columns to a word), in a
// tile-major layout whose word (t, g, r) holds columns of group g of tile row
// r at t * G * 64 + g * 64 + r (G = 32 or 64 groups per tile), so that the 64
// lanes' stores of one group are one coalesced 256-byte row.  Verbatim
// segments keep the placeholder index 0 (or its exponent); vrank[t][s][r]
// receives the index of segment s of tile row r in the verbatim store, or -1.
template <int PLAN, bool EXP>
__global__ __launch_bounds__(256) void k_transcode_bf16(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const LdsLayout L = lds_layout(1, a.max_words, true);
    const LaneCtx c = lane_ctx(a);
    const int S = a.max_words + 3;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + c.wave * S * 32;
    const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
    const LwTabRegs tr = lw_tab_fetch<PLAN>(a, !EXP);   // second table: the palette index itself
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
    const int r = 2 * c.l + c.half;                                   // tile row
    uint32_t *o = static_cast<uint32_t *>(a.out) + (size_t)c.t * (EXP ? 64 : 32) * 64 + r;
    struct NoAux {};
    uint32_t acc = 0;
    lw_decode_pipelined<PLAN, 64, NoAux, false>(
        d, a, [](int) { return EXP ? 0u : (LW_TPAY_HI - LW_TPAY); }, [](int) { return NoAux{}; },
        [&](int g, int j, uint32_t pay, const NoAux &) {
            if constexpr (EXP) {
                acc |= (pay >> 7) << (8 * j);                         // payload: exponent << 7
                if (j == 3) {
                    o[g * 64] = acc;
                    acc = 0;
                }
            } else {
                acc |= pay << (4 * (4 * (g & 1) + j));                 // payload: palette index
                if (j == 3 && (g & 1)) {
                    o[(g >> 1) * 64] = acc;
                    acc = 0;
                }
            }
        });
    // verbatim ranks of the tile, one row per lane (the walk is wave-uniform)
    const uint32_t mw = a.vb_bits[(size_t)c.t * 8 + (c.lane & 7)];
    uint32_t ord = a.vb_start[c.t];
    int32_t v[4] = {-1, -1, -1, -1};
    for (int w = 0; w < 8; w++) {
        uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)mw, w);
        while (bits) {
            const int bit = 32 * w + __builtin_ctz(bits);
            bits &= bits - 1u;
            const int row = bit >> 2, seg = bit & 3;
#pragma unroll
            for (int q = 0; q < 4; q++) v[q] = (c.lane == row && seg == q) ? (int32_t)ord : v[q];
            ord++;
        }
    }
#pragma unroll
    for (int q = 0; q < 4; q++) a.vrank[(size_t)c.t * 256 + q * 64 + c.lane] = v[q];
}

template <int PLAN, bool EXP>
hipError_t launch_transcode(const KArgs &a, hipStream_t s)
{
    const LdsLayout L = lds_layout(1, a.max_words, true);
    dim3 grid((unsigned)((a.n_cb + WAVES - 1) / WAVES), (unsigned)a.n_rb);
    hipError_t e = lw_allow_lds<k_transcode_bf16<PLAN, EXP>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_transcode_bf16<PLAN, EXP>), grid, dim3(256), L.total, s, a);
    return hipGetLastError();
}

template <int PLAN>
hipError_t transcode_mode(const KArgs &a, bool exponents, hipStream_t s)
{
    return exponents ? launch_transcode<PLAN, true>(a, s) : launch_transcode<PLAN, false>(a, s);
}

template <int PLAN, int BATCH, int WPG>
hipError_t launch_gemv_wpg(const KArgs &a0, hipStream_t s)
{
    KArgs a = a0;
    a.groups = (a.n_cb + WPG - 1) / WPG;  // column groups combined through the workspace (none if 1)
    a.ramp = lw_resident_ramp((int64_t)a.n_rb * a.n_cb);
    const LdsLayout L = lds_layout(BATCH, a.max_words, false, WPG);
    dim3 grid((unsigned)a.groups, (unsigned)a.n_rb);
    auto kern = k_gemv_bf16<PLAN, BATCH, WPG>;
    hipError_t e = lw_allow_lds<k_gemv_bf16<PLAN, BATCH, WPG>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(64 * WPG), L.total, s, a);
    return hipGetLastError();
}

// Whole rows (sixteen wavefronts) under the 4- and 6-bit kernels'
// conditions: 13..16 column blocks, at least 128 row bands, tiles in LDS.
template <int PLAN, int BATCH>
hipError_t launch_gemv(const KArgs &a, hipStream_t s)
{
    if constexpr (BATCH <= 4) {
        if (a.n_cb > 12 && a.n_cb <= 16 && a.n_rb >= 128 &&
            lds_layout(BATCH, a.max_words, false, 16).total <= (uint32_t)lw_device_lds_bytes())
            return launch_gemv_wpg<PLAN, BATCH, 16>(a, s);
    }
    return launch_gemv_wpg<PLAN, BATCH, WAVES>(a, s);
}

template <int PLAN>
hipError_t launch_decode(const KArgs &a0, hipStream_t s)
{
    KArgs a = a0;
    a.groups = (a.n_cb + WAVES - 1) / WAVES;
    const LdsLayout L = lds_layout(1, a.max_words, true);
    dim3 grid((unsigned)a.groups, (unsigned)a.n_rb);
    auto kern = k_decode_bf16<PLAN>;
    hipError_t e = lw_allow_lds<k_decode_bf16<PLAN>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(256), L.total, s, a);
    return hipGetLastError();
}

template <int PLAN>
hipError_t gemv_batch(const KArgs &a, int batch, hipStream_t s)
{
    switch (batch) {
    case 1: return launch_gemv<PLAN, 1>(a, s);
    case 2: return launch_gemv<PLAN, 2>(a, s);
    case 3: return launch_gemv<PLAN, 3>(a, s);
    case 4: return launch_gemv<PLAN, 4>(a, s);
    case 5: return launch_gemv<PLAN, 5>(a, s);
    case 6: return launch_gemv<PLAN, 6>(a, s);
    case 7: return launch_gemv<PLAN, 7>(a, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

hipError_t lw_launch_gemv_bf16(const KArgs &a, SadPlan p, int batch, hipStream_t s)
{
    return lw_with_plan(p, [&](auto P) { return gemv_batch<decltype(P)::value>(a, batch, s); });
}

hipError_t lw_launch_decode_bf16(const KArgs &a, SadPlan p, hipStream_t s)
{
    return lw_with_plan(p, [&](auto P) { return launch_decode<decltype(P)::value>(a, s); });
}

hipError_t lw_launch_transcode_bf16(const KArgs &a, SadPlan p, bool exponents, hipStream_t s)
{
    return lw_with_plan(p, [&](auto P) { return transcode_mode<decltype(P)::value>(a, exponents, s); });
}
