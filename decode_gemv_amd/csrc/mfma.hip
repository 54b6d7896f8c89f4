// mfma.hip -- fused decode + GEMM for batch 8..16 on the matrix cores of
// gfx950 ("LazyWeights" bundle, decoded as in lane_decode.hpp; the matrix
// product fed from on-chip memory follows the reconstructive matmul idea of
// "Unweight", section "How reconstructive matmul works").
//
// At batch >= 8 the product is a real dense contraction (64 rows x CHUNK
// columns x 16 batch per step), so the decoded weights go through a small
// LDS staging block into the matrix cores:
//   - one wavefront per tile: lane l + 32*half decodes tile row 2l + half
//     (the second row from its recorded start) and writes each group of
//     decoded weights into its row of a 64 x CHUNK staging block, the row's
//     four operand fragments permuted so that the stores (one fragment of 64
//     rows) and the fragment reads of the MFMA operands (16 rows x 4
//     fragments) each hit distinct banks;
//   - CHUNK = 32 columns (16-byte fragments, v_mfma_f32_16x16x32{f16,bf16})
//     where the workgroup's LDS holds the 4 KB blocks, else 16 (8-byte
//     fragments, v_mfma_f32_16x16x16{f16,bf16}); every CHUNK columns, 4 row
//     blocks accumulate D[row][batch] += W[row][k] * X[k][batch], with the X
//     fragments (x[batch][k], zero for batch >= the call's batch) loaded from
//     global memory one chunk ahead (loading all of them in the prologue
//     measured slower); the activation sums of the dequantisation come from
//     the same fragments by v_dot2 against (1, 1);
//   - dequantisation uses y = d * (W q x) - m * sum(x) per tile row.
// A workgroup is WPG wavefronts on WPG column blocks of one row band, as in
// the VALU kernel: sixteen (whole rows) when a row band has 13 to 16 column
// blocks, fourteen when the column blocks are a multiple of 14 and the whole
// grid is resident at once, else four.
// MFMA 16x16xK lane layout: A lane i = A[i%16][(K/4)(i/16) ..], B lane i =
// B[(K/4)(i/16) ..][i%16], D lane i = D[4(i/16)+j][i%16], j = 0..3.
#include <type_traits>

#include "lane_decode.hpp"

namespace {

constexpr int WAVES = 4;
constexpr int NB = 16;                     // batch columns of the MFMA tile
constexpr int RED_RS = 65;                 // floats per (wavefront, batch) run of the partial sums: the 16
                                           // lanes of one batch column store to distinct banks

// Columns staged per MFMA step: 16 (16x16x16 instructions, 8-byte operand
// fragments, 32-byte staged rows) or 32 (16x16x32, 16-byte fragments,
// 64-byte rows: half the matrix instructions and fragment reads, twice the
// staging block).
template <int CHUNK>
__host__ __device__ constexpr int stage_bytes() { return 64 * CHUNK * 2; }

// Byte offset of operand fragment f (columns f*CHUNK/4 .. +CHUNK/4-1) of
// staged row R.  Fragments are permuted within the row so that the 64 lanes'
// stores (one fragment of every row) and the operand reads (16 rows x 4
// fragments) each hit distinct banks, in 8-lane phases over 32 banks and in
// 16-lane phases over 64 (checked on the host for every store and read).
template <int CHUNK>
__host__ __device__ constexpr uint32_t stage_frag(int R, int f)
{
    if constexpr (CHUNK == 16)
        return (uint32_t)(R * 32 + 8 * (f ^ (((R >> 2) ^ (R >> 4)) & 3)));
    else
        return (uint32_t)(R * 64 + 16 * (f ^ (((R >> 1) ^ (R >> 3)) & 3)));
}

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct LdsLayout {
    uint32_t tiles, stage, flag, total;
};

// staged tiles: one per `parts` wavefronts; staging blocks: one per wavefront
__host__ __device__ inline LdsLayout lds_layout(int max_words, int waves, int chunk, int parts = 1)
{
    LdsLayout L;
    L.stage = LW_TAB_BYTES;
    L.tiles = L.stage + waves * 64 * chunk * 2;
    const uint32_t tiles = (uint32_t)((waves / parts) * (max_words + 3) * 128);
    const uint32_t red = (uint32_t)(waves * NB * RED_RS * 4);
    L.flag = L.tiles + (tiles > red ? tiles : red);
    L.total = L.flag + 16;
    return L;
}

// Identity of a lane: wavefront w decodes part w % parts of the tile in slot
// w / parts; lane l + 32*half decodes that part of tile row 2l + half; the
// lane's index is also its row of the staged weight block.
struct LaneCtx {
    int wave, lane, half, l, g, cb, rb, t, ts, p;
    bool active;
};

LW_DEV LaneCtx lane_ctx(const KArgs &a, int waves, int parts)
{
    LaneCtx c;
    c.wave = (int)lw_wave_id();
    c.lane = threadIdx.x & 63;
    c.half = c.lane >> 5;
    c.l = c.lane & 31;
    c.g = blockIdx.x;
    c.rb = blockIdx.y;
    c.ts = c.wave / parts;
    c.p = c.wave % parts;
    c.cb = c.g * (waves / parts) + c.ts;
    c.active = c.cb < a.n_cb;
    c.t = c.rb * a.n_cb + (c.active ? c.cb : 0);
    return c;
}

LW_DEV void lw_st64(uint32_t addr, u32x2 v) { *(__attribute__((address_space(3))) u32x2 *)(size_t)addr = v; }
LW_DEV void lw_st128(uint32_t addr, u32x4 v) { *(__attribute__((address_space(3))) u32x4 *)(size_t)addr = v; }
LW_DEV u32x2 lw_ld64(uint32_t addr) { return *(__attribute__((address_space(3))) const u32x2 *)(size_t)addr; }
LW_DEV u32x4 lw_ld128(uint32_t addr) { return *(__attribute__((address_space(3))) const u32x4 *)(size_t)addr; }

// One 16x16 block of D += A B over a chunk: 16x16x16 on 8-byte fragments or
// 16x16x32 on 16-byte ones.
template <int KIND>
LW_DEV f4 mfma(u32x2 a, u32x2 b, f4 acc)
{
    if constexpr (KIND == LW_BF16_EXP)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), acc, 0,
                                                          0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, b), acc, 0, 0, 0);
}

template <int KIND>
LW_DEV f4 mfma(u32x4 a, u32x4 b, f4 acc)
{
    if constexpr (KIND == LW_BF16_EXP)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), acc, 0, 0,
                                                       0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), acc, 0, 0, 0);
}

// P parts per tile row (bundles in parts, 4- and 6-bit): each wavefront
// decodes and multiplies one part's columns; the parts of a tile share its
// staged words, as in fused_q.hip.
template <int KIND, int PLAN, int WPG, int CHUNK, int P>
__global__ __launch_bounds__(64 * WPG) void k_gemv_mfma(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    static_assert(CHUNK == 16 || CHUNK == 32, "16- or 32-column steps");
    static_assert(P == 1 || KIND != LW_BF16_EXP, "bf16 tiles are decoded in whole rows");
    static_assert(WPG % P == 0, "whole tiles per workgroup");
    typedef typename std::conditional<CHUNK == 16, u32x2, u32x4>::type frag;   // one lane's operand fragment
    constexpr int FW = CHUNK / 8;                          // 32-bit words per fragment
    constexpr int GPC = (KIND == LW_Q4_PAIR ? 2 : 4) * (CHUNK / 16);   // groups of four symbols per chunk
    constexpr int NG = (KIND == LW_Q4_PAIR ? 32 : 64) / P;   // groups per part of a tile row
    constexpr int NCHUNK = 256 / CHUNK / P;                // chunks per part
    static_assert(NG % GPC == 0, "whole chunks per part");
    const LdsLayout L = lds_layout(a.max_words, WPG, CHUNK, P);
    const LaneCtx c = lane_ctx(a, WPG, P);
    const int S = a.max_words + 3;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + c.ts * S * 32;
    const uint32_t stage = (uint32_t)(size_t)(lds + L.stage + c.wave * stage_bytes<CHUNK>());
    // MFMA fragment coordinates of this lane
    const int fr = c.lane & 15, fk = c.lane >> 4;
    // this lane's stores (fragment f of row lane) and operand reads (fragment fk of row 16 r + fr)
    uint32_t st_at[4], ld_at[4];
#pragma unroll
    for (int f = 0; f < 4; f++) {
        st_at[f] = stage + stage_frag<CHUNK>(c.lane, f);
        ld_at[f] = stage + stage_frag<CHUNK>(16 * f + fr, fk);
    }

    // issue every load, tile offsets first; table barrier; own tile (as in fused_q.hip)
    const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
    const LwTabRegs tr = lw_tab_fetch<lw_compact<PLAN>()>(a, false);
    // this lane's part: bundle part half * parts + p * (parts / P)
    const uint32_t start = lw_part_start(a, c.t, c.l, c.half * a.parts + c.p * (a.parts / P));
    LwTileRegs64 tile;
    if constexpr (P > 1) {
        // the tile's first wavefront stages it; one barrier covers the table and the tiles
        if (c.p == 0) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        lw_tab_put<lw_compact<PLAN>()>(lds, tr, a);
        if (c.p == 0) lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        __syncthreads();
    } else {
        if constexpr (WPG <= WAVES) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        lw_tab_put<lw_compact<PLAN>()>(lds, tr, a);
        __syncthreads();                  // the decoder table is complete
        if constexpr (WPG > WAVES) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    }

    // x fragments: lane holds x[b = fr][col0 + CHUNK chunk + (CHUNK/4) fk ..] of this part's
    // columns, zero for b >= batch
    const bool xb_ok = fr < a.batch;
    const uint16_t *xrow = a.x + (size_t)(xb_ok ? fr : 0) * a.cols + (size_t)(c.active ? c.cb : 0) * 256 +
                           CHUNK * NCHUNK * c.p + (CHUNK / 4) * fk;
    auto load_x = [&](int chunk) -> frag {
        const frag v = *reinterpret_cast<const frag *>(xrow + CHUNK * chunk);
        return xb_ok ? v : frag{};
    };

    f4 acc[4];
#pragma unroll
    for (int r = 0; r < 4; r++) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
    float sx = 0.f;                          // sum of x[fr][k] over this lane's k subset

    if (c.active) {
        LaneDec d;
        const bool ok = lw_lane_init(d, lds, slots, c.l, a);
        d.advance(start);
        if (ok) {
            frag xcur = load_x(0);
            uint32_t gw[4];                   // the current group's 16-bit weights, two per word
            // A chunk's weight fragments are requested when its last group is
            // stored and multiplied one group later, so the LDS round trip
            // overlaps decoding (the next group's store to the same staging
            // row is issued after those reads, and a wavefront's LDS
            // operations complete in order).
            frag af[4], xpend;
            auto read_chunk = [&](int chunk) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    if constexpr (CHUNK == 16) af[r] = lw_ld64(ld_at[r]);
                    else af[r] = lw_ld128(ld_at[r]);
                }
                xpend = xcur;
                // x of the next chunk, used one chunk of decoding later
                xcur = load_x(chunk + 1 < NCHUNK ? chunk + 1 : chunk);
            };
            auto mfma_step = [&]() {
#pragma unroll
                for (int w = 0; w < FW; w++) {
                    if constexpr (KIND == LW_BF16_EXP)
                        sx += __builtin_bit_cast(float, xpend[w] << 16) + __builtin_bit_cast(float, xpend[w] & 0xFFFF0000u);
                    else
                        sx = lw_dot2(xpend[w], 0x3C003C00u, sx);     // (1, 1) in fp16
                }
#pragma unroll
                for (int r = 0; r < 4; r++) acc[r] = mfma<KIND>(af[r], xpend, acc[r]);
            };
            auto put = [&](int g, int j, uint32_t pay, uint32_t smw) {
                if (j == 0) lw_ramp<NG>(a.ramp, g);
                // 16-bit weights of this symbol into the group's words
                if constexpr (KIND == LW_Q4_PAIR) {
                    gw[j] = pay;
                } else if constexpr (KIND == LW_BF16_EXP) {
                    if (j & 1) {
                        const uint32_t spread = __builtin_amdgcn_perm(smw, smw, j == 1 ? 0x01010000u : 0x03030202u);
                        gw[j >> 1] = (spread & 0x807F807Fu) | gw[j >> 1] | pay;
                    } else {
                        gw[j >> 1] = pay;
                    }
                } else {
                    if (j & 1) gw[j >> 1] |= pay;
                    else gw[j >> 1] = pay;
                }
                if (j == 3) {
                    // the group's weights into the staged row: Q4 8 columns (two 8-byte
                    // fragments, or one 16-byte), Q6 and bf16 4 columns (one 8-byte
                    // fragment, or half a 16-byte one)
                    if constexpr (CHUNK == 16) {
                        if constexpr (KIND == LW_Q4_PAIR) {
                            lw_st64(st_at[2 * (g % GPC)], u32x2{gw[0], gw[1]});
                            lw_st64(st_at[2 * (g % GPC) + 1], u32x2{gw[2], gw[3]});
                        } else {
                            lw_st64(st_at[g % GPC], u32x2{gw[0], gw[1]});
                        }
                    } else {
                        if constexpr (KIND == LW_Q4_PAIR)
                            lw_st128(st_at[g % GPC], u32x4{gw[0], gw[1], gw[2], gw[3]});
                        else
                            lw_st64(st_at[(g % GPC) >> 1] + 8u * (uint32_t)(g & 1), u32x2{gw[0], gw[1]});
                    }
                    if ((g % GPC) == 0 && g > 0) mfma_step();          // the previous chunk
                    if ((g % GPC) == GPC - 1) read_chunk(g / GPC);
                }
            };
            auto pay_off = [](int j) { return (KIND != LW_Q4_PAIR && (j & 1)) ? (LW_TPAY_HI - LW_TPAY) : 0u; };
            if constexpr (KIND == LW_BF16_EXP) {
                // sign+mantissa words stream in 16-group chunks, as in the VALU kernel
                const uint32_t *smrow = a.sm + (size_t)c.t * 4096 + (size_t)c.half * 64 * 32 + c.l;
                struct XA {
                    uint32_t sm;
                };
                uint32_t ring[2][16];
                auto run_chunk = [&](int ch, const uint32_t (&cur)[16]) {
                    lw_decode_pipelined<PLAN, 16, XA, true>(
                        d, a, pay_off, [&](int g) { return XA{cur[g]}; },
                        [&](int g, int j, uint32_t pay, const XA &x) { put(16 * ch + g, j, pay, x.sm); });
                };
#pragma unroll
                for (int i = 0; i < 16; i++) ring[0][i] = smrow[i * 32];
#pragma unroll
                for (int ch = 0; ch < 4; ch += 2) {
#pragma unroll
                    for (int i = 0; i < 16; i++) ring[1][i] = smrow[((ch + 1) * 16 + i) * 32];
                    run_chunk(ch, ring[0]);
                    if (ch + 2 < 4)
#pragma unroll
                        for (int i = 0; i < 16; i++) ring[0][i] = smrow[((ch + 2) * 16 + i) * 32];
                    run_chunk(ch + 1, ring[1]);
                }
            } else {
                struct NoAux {};
                lw_decode_pipelined<PLAN, NG, NoAux, true>(
                    d, a, pay_off, [](int) { return NoAux{}; },
                    [&](int g, int j, uint32_t pay, const NoAux &) { put(g, j, pay, 0u); });
            }
            mfma_step();                      // the last chunk
        } else {
#pragma unroll
            for (int r = 0; r < 4; r++)
                acc[r] = f4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        }
    }
    // sum of x over the tile's 256 columns for batch column fr
    sx += __shfl_xor(sx, 16, 64);
    sx += __shfl_xor(sx, 32, 64);

    __syncthreads();                      // tiles no longer read: reuse for the reduction
    float *red = reinterpret_cast<float *>(lds + L.tiles);
    // D lane layout: staged row R = 16 r + 4 fk + jj (= wavefront lane R, which
    // decoded tile row 2 (R % 32) + R / 32), batch column fr
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const int R = 16 * r + 4 * fk + jj;
            const int trow = 2 * (R & 31) + (R >> 5);
            float v = 0.f;
            if (c.active) {
                if constexpr (KIND == LW_BF16_EXP) {
                    v = acc[r][jj];              // bf16 bundles carry no scales
                } else {
                    const uint32_t w = a.dm[(size_t)c.t * 64 + trow];
                    v = lw_half_lo(w) * acc[r][jj] - lw_half_hi(w) * sx;
                }
            }
            red[(c.wave * NB + fr) * RED_RS + trow] = v;
        }
    __syncthreads();
    if constexpr (KIND == LW_BF16_EXP) {
        // verbatim segments (rare): replace the placeholder weights'
        // contribution by the stored values', all lanes on one segment; lane
        // 0 adds each batch column's sum to this wavefront's partial rows
        if (c.active) {
            const uint16_t *xcol = a.x + (size_t)c.cb * 256;
            lw_verbatim_visit(a, c.t, c.lane, [&](int row, int col, uint32_t vv, uint32_t ph) {
                const float wdiff = __builtin_bit_cast(float, vv << 16) - __builtin_bit_cast(float, ph << 16);
                for (int b = 0; b < a.batch; b++) {
                    const float sb = lw_wave_sum(
                        wdiff * __builtin_bit_cast(float, (uint32_t)xcol[(size_t)b * a.cols + col] << 16));
                    if (c.lane == 0) red[(c.wave * NB + b) * RED_RS + row] += sb;
                }
            });
        }
        __syncthreads();
    }
    uint32_t *last_flag = reinterpret_cast<uint32_t *>(lds + L.flag);
    lw_finish_rows<NB, 64, RED_RS>(a, red, (int64_t)c.rb * 64, c.g, c.rb, WPG, last_flag);
}

template <int KIND, int PLAN, int WPG, int CHUNK, int P = 1>
hipError_t launch_wpg(const KArgs &a0, hipStream_t s)
{
    KArgs a = a0;
    constexpr int TPW = WPG / P;          // column blocks per workgroup
    a.groups = (a.n_cb + TPW - 1) / TPW;  // column groups combined through the workspace (none if 1)
    if (a.groups > 1 && a.groups > lw_work_groups(a.n_cb, a.parts)) return hipErrorInvalidValue;
    a.ramp = lw_resident_ramp((int64_t)a.n_rb * a.n_cb * P);
    const LdsLayout L = lds_layout(a.max_words, WPG, CHUNK, P);
    dim3 grid((unsigned)a.groups, (unsigned)a.n_rb);
    auto kern = k_gemv_mfma<KIND, PLAN, WPG, CHUNK, P>;
    hipError_t e = lw_allow_lds<k_gemv_mfma<KIND, PLAN, WPG, CHUNK, P>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(64 * WPG), L.total, s, a);
    return hipGetLastError();
}

// Workgroup shape as in the VALU kernel: whole rows (16 wavefronts) for 13..16
// column blocks and at least 128 row bands, 14 wavefronts when the column
// blocks are a multiple of 14 and the whole grid is resident at once, when
// the staged tiles fit in LDS; else four.  32-column steps wherever their
// staging blocks fit (the whole-row layout takes 16).
template <int KIND, int PLAN>
hipError_t launch(const KArgs &a, hipStream_t s)
{
    const uint32_t lds = (uint32_t)lw_device_lds_bytes();
    if constexpr (KIND != LW_BF16_EXP) {
        // bundles in parts: eight-wavefront workgroups, as the VALU kernel
        if (a.parts == 2 && lds_layout(a.max_words, 8, 32, 2).total <= lds) return launch_wpg<KIND, PLAN, 8, 32, 2>(a, s);
        if (a.parts == 4 && lds_layout(a.max_words, 8, 32, 4).total <= lds) return launch_wpg<KIND, PLAN, 8, 32, 4>(a, s);
        if (a.parts == 8 && lds_layout(a.max_words, 8, 32, 8).total <= lds) return launch_wpg<KIND, PLAN, 8, 32, 8>(a, s);
    }
    if (a.n_cb > 12 && a.n_cb <= 16 && a.n_rb >= 128 && lds_layout(a.max_words, 16, 16).total <= lds)
        return launch_wpg<KIND, PLAN, 16, 16>(a, s);
    if (a.n_cb > 16 && a.n_cb % 14 == 0 && lw_resident_ramp((int64_t)a.n_rb * a.n_cb)) {
        if (lds_layout(a.max_words, 14, 32).total <= lds) return launch_wpg<KIND, PLAN, 14, 32>(a, s);
        if (lds_layout(a.max_words, 14, 16).total <= lds) return launch_wpg<KIND, PLAN, 14, 16>(a, s);
    }
    return launch_wpg<KIND, PLAN, WAVES, 32>(a, s);
}

template <int KIND>
hipError_t by_plan(const KArgs &a, SadPlan p, hipStream_t s)
{
    return lw_with_plan(p, [&](auto P) { return launch<KIND, decltype(P)::value>(a, s); });
}

}  // namespace

hipError_t lw_launch_gemv_mfma(const KArgs &a, int kind, SadPlan p, int batch, hipStream_t s)
{
    if (batch < 1 || batch > NB) return hipErrorInvalidValue;
    if (kind == LW_Q4_PAIR) return by_plan<LW_Q4_PAIR>(a, p, s);
    if (kind == LW_Q6_SINGLE) return by_plan<LW_Q6_SINGLE>(a, p, s);
    if (kind == LW_BF16_EXP) return by_plan<LW_BF16_EXP>(a, p, s);
    return hipErrorInvalidValue;
}
