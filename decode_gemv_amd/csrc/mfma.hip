// mfma.hip -- fused decode + GEMM for batch 8..16 on the matrix cores of
// gfx950 ("LazyWeights" bundle, decoded as in lane_decode.hpp; feeding the
// matrix cores from on-chip data follows the reconstructive matmul idea of
// "Unweight", section "How reconstructive matmul works").
//
// At batch >= 8 the product is a real dense contraction, and a lane's decoded
// weights are already a matrix-core operand.  Lane l + 32*half decodes tile
// row 2l + half (one wavefront per part of a tile, as in fused_q.hip); after
// one group of four symbols (4-bit pairs) or two (6-bit codes, bf16
// exponents) it holds that row's weights at 8 consecutive columns, which is
// exactly its B operand of v_mfma_f32_32x32x16_{f16,bf16} for B[k][n], n = l,
// k = 8*half + e.  The activations go in as a block-diagonal A:
//   A[2b + h][8h' + e] = x[b][col + e] when h == h', else 0,
// so D[2b + h][n] accumulates x[b] . W[row 2n + h]: batch row b against both
// rows of the lane pair.  One matrix instruction per 8 columns replaces any
// staging of the decoded weights through LDS; half of A is zero, which the
// matrix cores absorb (a 32x32x16 per 8 columns is about a tenth of the
// SIMD's issue time for decoding them).  Each lane fetches its A fragments
// straight from global memory, 16 bytes (8 columns) a load, three or four
// groups ahead (lanes off the diagonal, and batch rows past the call's batch,
// read a line of zeros).
// MFMA 32x32x16 lane layout: A lane i = A[i%32][8(i/32) ..], B lane i =
// B[8(i/32) ..][i%32], D lane i register j = D[8(j/4) + 4(i/32) + j%4][i%32].
//
// Dequantisation (4- and 6-bit) uses y = d * (W q x) - m * sum(x) per tile
// row; the activation sums come from the A fragments as they pass (4-bit) or
// from one read of the part's activations in the prologue (6-bit, whose
// decode is twice as long per column).  bf16 weights need no dequantisation;
// their verbatim segments are corrected after the decode, as in the VALU
// kernel.  Workgroups have the VALU kernel's shapes: eight wavefronts on
// bundles in parts, sixteen (whole rows) for 13 to 16 column blocks and at
// least 128 row bands, fourteen when the column blocks are a multiple of 14
// and the whole grid is resident at once, else four (a balanced layout as in
// fused_q.hip measured no faster at batch 8 and 16: 24.7-25.0 against 25.0 us
// on 4096x14336).
#include <type_traits>

#include "lane_decode.hpp"

namespace {

constexpr int WAVES = 4;
constexpr int NB = 16;                     // batch rows of the matrix-core tile
constexpr int RED_RS = 65;                 // floats per (wavefront, batch) run of the partial sums

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f16x __attribute__((ext_vector_type(16)));   // one lane's 32x32 accumulator block
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Activations for lanes off the A operand's diagonal: one part of a tile
// row's columns, 512 bytes, never written.
__device__ __attribute__((aligned(16))) uint32_t lw_zero_x[128] = {};

// D += A B on 16-byte fragments: eight columns of fp16 (4- and 6-bit codes)
// or bf16 weights
template <int KIND>
LW_DEV f16x mfma32(u32x4 a, u32x4 b, f16x acc)
{
    if constexpr (KIND == LW_BF16_EXP)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), acc, 0, 0, 0);
}

struct LdsLayout {
    uint32_t tiles, total;
};

// the decoder table, then the staged tiles (one per `parts` wavefronts),
// reused for the per-wavefront partial sums once decoding is done
__host__ __device__ inline LdsLayout lds_layout(int max_words, int waves, int parts)
{
    LdsLayout L;
    L.tiles = LW_TAB_BYTES;
    const uint32_t tiles = (uint32_t)((waves / parts) * (max_words + 3) * 128);
    const uint32_t red = (uint32_t)(waves * NB * RED_RS * 4);
    L.total = L.tiles + (tiles > red ? tiles : red);
    return L;
}

// Identity of a lane: wavefront w decodes part w % parts of the tile in slot
// w / parts; lane l + 32*half decodes that part of tile row 2l + half.
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

template <int KIND, int PLAN, int WPG, int P>
__global__ __launch_bounds__(64 * WPG) void k_gemv_mfma(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    static_assert(WPG % P == 0, "whole tiles per workgroup");
    static_assert(P == 1 || KIND != LW_BF16_EXP, "bf16 tiles are decoded in whole rows");
    constexpr bool Q4 = KIND == LW_Q4_PAIR, BF = KIND == LW_BF16_EXP;
    constexpr int NG = (Q4 ? 32 : 64) / P;   // groups of four symbols per part of a tile row
    constexpr int PCOLS = 256 / P;           // columns per part
    constexpr int GPL = Q4 ? 1 : 2;          // groups per matrix instruction and per 16-byte activation load
    constexpr int NL = NG / GPL;             // activation loads per part
    constexpr int DIST = Q4 ? 3 : 2;         // loads between an A fragment's load and its first use
    const LdsLayout L = lds_layout(a.max_words, WPG, P);
    const LaneCtx c = lane_ctx(a, WPG, P);
    const int S = a.max_words + 3;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + c.ts * S * 32;

    // Issue every global load first, tile offsets first (as in fused_q.hip).
    const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
    const LwTabRegs tr = lw_tab_fetch<PLAN>(a, false);
    const uint32_t start = lw_part_start(a, c.t, c.l, c.half * a.parts + c.p * (a.parts / P));
    // (d, m) of tile rows 2l and 2l + 1, the two rows of this lane's D column
    u32x2 dm2 = u32x2{0u, 0u};
    if constexpr (!BF) dm2 = *reinterpret_cast<const u32x2 *>(a.dm + (size_t)c.t * 64 + 2 * c.l);
    const size_t col0 = (size_t)(c.active ? c.cb : 0) * 256 + (size_t)PCOLS * c.p;
    // Activation sums of the dequantisation.  Q4: the diagonal lanes add
    // their A fragments as they pass (four v_dot2 a group, against reading
    // the part's activations once more up front, which holds back the first
    // tile by about 2 us); Q6 adds them in the prologue: lane i takes batch
    // row i/4 over quarter i%4 of the part's columns.
    constexpr bool SX_PRO = KIND == LW_Q6_SINGLE;
    constexpr int SQW = SX_PRO ? PCOLS / 4 / 8 : 1;   // 16-byte words per quarter
    u32x4 sv[SQW];
    if constexpr (SX_PRO) {
        const int sb = c.lane >> 2, sq = c.lane & 3;
        const u32x4 *sp = sb < a.batch
                              ? reinterpret_cast<const u32x4 *>(a.x + (size_t)sb * a.cols + col0 + sq * (PCOLS / 4))
                              : reinterpret_cast<const u32x4 *>(lw_zero_x);
#pragma unroll
        for (int i = 0; i < SQW; i++) sv[i] = sp[i];
    }
    LwTileRegs64 tile;
    if constexpr (P > 1) {
        // the tile's first wavefront stages it; one barrier covers the table and the tiles
        if (c.p == 0) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        lw_tab_put<PLAN>(lds, tr, a);
        if (c.p == 0) lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        __syncthreads();
    } else {
        if constexpr (WPG <= WAVES) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        lw_tab_put<PLAN>(lds, tr, a);
        __syncthreads();                  // the decoder table is complete
        if constexpr (WPG > WAVES) lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
        lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    }
    // Q4: this lane's A fragments summed (batch row l/2 at lane l, l even);
    // Q6: in every lane of quad b, batch row b's sum
    float sxq = 0.f;
    if constexpr (SX_PRO) {
#pragma unroll
        for (int i = 0; i < SQW; i++)
#pragma unroll
            for (int w = 0; w < 4; w++) sxq = lw_dot2(sv[i][w], 0x3C003C00u, sxq);   // (1, 1) in fp16
        sxq = lw_group_sum<4>(sxq);
    }

    // this lane's A fragments: batch row l/2 on the diagonal (l % 2 == half),
    // else zeros; loaded 16 bytes at a time (one group's Q4 fragment, two
    // groups' Q6 or bf16 ones)
    const int xb = c.l >> 1;
    const bool diag = (c.l & 1) == c.half && xb < a.batch;
    const u32x4 *xp = diag ? reinterpret_cast<const u32x4 *>(a.x + (size_t)xb * a.cols + col0)
                           : reinterpret_cast<const u32x4 *>(lw_zero_x);

    f16x acc = {};
    if (c.active) {
        LaneDec d;
        const bool ok = lw_lane_init(d, lds, slots, c.l, a);
        d.advance(start);
        if (ok) {
            u32x4 xr[DIST + 1];           // ring of activation loads, indexed by load (a compile-time constant)
#pragma unroll
            for (int q = 0; q < DIST; q++) xr[q] = xp[q];
            uint32_t gw[4];               // eight columns' weights, two 16-bit ones per word
            // A group's weights into the B fragment; after the last group of
            // a fragment (every group for Q4, every second one for Q6 and
            // bf16), the matrix instruction with its A fragment.
            // pay: the symbol's payload (Q4 a pair of fp16 codes; Q6 one
            // fp16 code, in the low half for even symbols and the high half
            // for odd ones; bf16 the exponent bits, placed likewise); smw:
            // bf16 sign+mantissa bytes of the group's four columns.
            auto put = [&](int g, int j, uint32_t pay, uint32_t smw, const u32x4 &xv) {
                if constexpr (Q4) {
                    gw[j] = pay;
                } else {
                    const int w = 2 * (g & 1) + (j >> 1);
                    if constexpr (BF) {
                        if (j & 1) {
                            const uint32_t spread = __builtin_amdgcn_perm(smw, smw, j == 1 ? 0x01010000u : 0x03030202u);
                            gw[w] = (spread & 0x807F807Fu) | gw[w] | pay;
                        } else {
                            gw[w] = pay;
                        }
                    } else {
                        if (j & 1) gw[w] |= pay;
                        else gw[w] = pay;
                    }
                }
                if (j == 3 && g % GPL == GPL - 1) {
                    acc = mfma32<KIND>(xv, u32x4{gw[0], gw[1], gw[2], gw[3]}, acc);
                    if constexpr (Q4) {
#pragma unroll
                        for (int w = 0; w < 4; w++) sxq = lw_dot2(xv[w], 0x3C003C00u, sxq);
                    }
                }
            };
            // the A fragment of group g (loaded DIST loads earlier); at the
            // first group of a load, issues the load DIST further on
            auto next_x = [&](int g) -> u32x4 {
                lw_ramp<NG>(a.ramp, g);
                const int q = g / GPL;
                if (g % GPL == 0 && q + DIST < NL) xr[(q + DIST) % (DIST + 1)] = xp[q + DIST];
                return xr[q % (DIST + 1)];
            };
            auto pay_off = [](int j) { return (!Q4 && (j & 1)) ? (LW_TPAY_HI - LW_TPAY) : 0u; };
            if constexpr (BF) {
                // sign+mantissa words stream in 16-group chunks, as in the VALU kernel
                const uint32_t *smrow = a.sm + (size_t)c.t * 4096 + (size_t)c.half * 64 * 32 + c.l;
                struct XA {
                    u32x4 x;
                    uint32_t sm;
                };
                uint32_t ring[2][16];
                auto run_chunk = [&](int ch, const uint32_t (&cur)[16]) {
                    lw_decode_pipelined<PLAN, 16, XA, true>(
                        d, a, pay_off, [&](int g) { return XA{next_x(16 * ch + g), cur[g]}; },
                        [&](int g, int j, uint32_t pay, const XA &x) { put(16 * ch + g, j, pay, x.sm, x.x); });
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
                struct XA {
                    u32x4 x;
                };
                lw_decode_pipelined<PLAN, NG, XA, true>(
                    d, a, pay_off, [&](int g) { return XA{next_x(g)}; },
                    [&](int g, int j, uint32_t pay, const XA &x) { put(g, j, pay, 0u, x.x); });
            }
        } else {                           // unusable LDS base: poison the output
#pragma unroll
            for (int j = 0; j < 16; j++) acc[j] = __builtin_nanf("");
        }
    }

    __syncthreads();                      // tiles no longer read: reuse for the partial sums
    float *red = reinterpret_cast<float *>(lds + L.tiles);
    // red[wave][b][row]: register j holds batch row b = D row / 2 against tile row 2l + (j & 1)
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int b = 4 * (j >> 2) + 2 * c.half + ((j & 3) >> 1);
        float v = 0.f;
        if constexpr (BF) {
            v = c.active ? acc[j] : 0.f;  // bf16 bundles carry no scales
        } else {
            const float sx = __shfl(sxq, SX_PRO ? 4 * b : 2 * b, 64);
            const uint32_t w = (j & 1) ? dm2.y : dm2.x;
            v = c.active ? lw_half_lo(w) * acc[j] - lw_half_hi(w) * sx : 0.f;
        }
        red[(c.wave * NB + b) * RED_RS + 2 * c.l + (j & 1)] = v;
    }
    __syncthreads();
    if constexpr (BF) {
        // verbatim segments (rare): replace the placeholder weights'
        // contribution by the stored values', all lanes on one segment; lane
        // 0 adds each batch row's sum to this wavefront's partial rows
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
    lw_finish_rows<NB, 64, RED_RS>(a, red, (int64_t)c.rb * 64, c.g, WPG);
}

template <int KIND, int PLAN, int WPG, int P>
hipError_t launch_wpg(const KArgs &a0, hipStream_t s)
{
    KArgs a = a0;
    constexpr int TPW = WPG / P;          // column blocks per workgroup
    a.groups = (a.n_cb + TPW - 1) / TPW;  // column groups combined through the workspace (none if 1)
    if (a.groups > 1 && a.groups > lw_work_groups(a.n_cb, a.parts)) return hipErrorInvalidValue;
    a.ramp = lw_resident_ramp((int64_t)a.n_rb * a.n_cb * P);
    const LdsLayout L = lds_layout(a.max_words, WPG, P);
    dim3 grid((unsigned)a.groups, (unsigned)a.n_rb);
    auto kern = k_gemv_mfma<KIND, PLAN, WPG, P>;
    hipError_t e = lw_allow_lds<k_gemv_mfma<KIND, PLAN, WPG, P>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(64 * WPG), L.total, s, a);
    return hipGetLastError();
}

template <int KIND, int PLAN>
hipError_t launch(const KArgs &a, hipStream_t s)
{
    const uint32_t lds = (uint32_t)lw_device_lds_bytes();
    if constexpr (KIND != LW_BF16_EXP) {
        // part layouts for the bundles in parts for their size, as the VALU kernel
        if ((int64_t)a.n_rb * a.n_cb * a.parts <= LW_PART_UNITS) {
            if (a.parts == 2 && lds_layout(a.max_words, 8, 2).total <= lds) return launch_wpg<KIND, PLAN, 8, 2>(a, s);
            if (a.parts == 4 && lds_layout(a.max_words, 8, 4).total <= lds) return launch_wpg<KIND, PLAN, 8, 4>(a, s);
            if (a.parts == 8 && lds_layout(a.max_words, 8, 8).total <= lds) return launch_wpg<KIND, PLAN, 8, 8>(a, s);
        }
    }
    if (a.n_cb > 12 && a.n_cb <= 16 && a.n_rb >= 128 && lds_layout(a.max_words, 16, 1).total <= lds)
        return launch_wpg<KIND, PLAN, 16, 1>(a, s);
    if (a.n_cb > 16 && a.n_cb % 14 == 0 && lw_resident_ramp((int64_t)a.n_rb * a.n_cb) &&
        lds_layout(a.max_words, 14, 1).total <= lds)
        return launch_wpg<KIND, PLAN, 14, 1>(a, s);
    return launch_wpg<KIND, PLAN, WAVES, 1>(a, s);
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
