// mfma.hip -- fused decode + GEMM for batch 8..16 on the matrix cores of
// gfx950 ("LazyWeights" bundle, decoded as in lane_decode.hpp; the matrix
// product fed from on-chip memory follows the reconstructive matmul idea of
// "Unweight", section "How reconstructive matmul works").
//
// At batch >= 8 the product is a real dense contraction (64 rows x 32
// columns x 16 batch per step), so the decoded weights go through a small
// LDS staging tile into v_mfma_f32_16x16x16{f16,bf16}:
//   - one wavefront per tile: lane l + 32*half decodes tile row 2l + half
//     (the second row from the lane's split bit) 32 columns at a time and
//     writes them as 16-bit values to stage[lane][0..31] (row stride 80
//     bytes: conflict-free 16-byte writes and 8-byte fragment reads);
//   - every 32 columns, 2 k-steps x 4 row blocks of 16x16x16 MFMA
//     accumulate D[row][batch] += W[row][k] * X[k][batch], with the X
//     fragments (x[batch][k], zero for batch >= the call's batch) loaded
//     from global memory one chunk ahead;
//   - dequantisation uses y = d * (W q x) - m * sum(x) per tile row.
// MFMA 16x16x16 lane layout: A lane i = A[i%16][4(i/16)..+3], B lane i =
// B[4(i/16)..+3][i%16], D lane i = D[4(i/16)+j][i%16], j = 0..3.
#include <type_traits>

#include "lane_decode.hpp"

namespace {

constexpr int WAVES = 4;
constexpr int NB = 16;                     // batch columns of the MFMA tile
constexpr int STAGE_STRIDE = 80;           // bytes per staged row (32 x 2 bytes + 16 pad)
constexpr int STAGE_BYTES = 64 * STAGE_STRIDE;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct LdsLayout {
    uint32_t tiles, stage, flag, total;
};

__host__ __device__ inline LdsLayout lds_layout(int max_words)
{
    LdsLayout L;
    L.stage = LW_TAB_BYTES;
    L.tiles = L.stage + WAVES * STAGE_BYTES;
    const uint32_t tiles = (uint32_t)(WAVES * (max_words + 3) * 128);
    const uint32_t red = (uint32_t)(WAVES * NB * 64 * 4);
    L.flag = L.tiles + (tiles > red ? tiles : red);
    L.total = L.flag + 16;
    return L;
}

// Identity of a lane: one wavefront per tile, lane l + 32*half decodes tile
// row 2l + half (the second row from the lane's split bit); the lane's index
// is also its row of the staged 64 x 32 weight block.
struct LaneCtx {
    int wave, lane, half, l, g, cb, rb, t;
    bool active;
};

LW_DEV LaneCtx lane_ctx(const KArgs &a)
{
    LaneCtx c;
    c.wave = (int)lw_wave_id();
    c.lane = threadIdx.x & 63;
    c.half = c.lane >> 5;
    c.l = c.lane & 31;
    c.g = blockIdx.x;
    c.rb = blockIdx.y;
    c.cb = c.g * WAVES + c.wave;
    c.active = c.cb < a.n_cb;
    c.t = c.rb * a.n_cb + (c.active ? c.cb : 0);
    return c;
}

LW_DEV void lw_st32(uint32_t addr, uint32_t v) { *(__attribute__((address_space(3))) uint32_t *)(size_t)addr = v; }
LW_DEV u32x2 lw_ld64(uint32_t addr) { return *(__attribute__((address_space(3))) const u32x2 *)(size_t)addr; }

template <int KIND>
LW_DEV f4 mfma(u32x2 a, u32x2 b, f4 acc)
{
    if constexpr (KIND == LW_BF16_EXP)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), acc, 0,
                                                          0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, b), acc, 0, 0, 0);
}

template <int KIND, int PLAN>
__global__ __launch_bounds__(256) void k_gemv_mfma(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int GPC = KIND == LW_Q4_PAIR ? 4 : 8;      // groups of four symbols per 32-column chunk
    constexpr int NG = KIND == LW_Q4_PAIR ? 32 : 64;     // groups per tile row
    const LdsLayout L = lds_layout(a.max_words);
    const LaneCtx c = lane_ctx(a);
    const int S = a.max_words + 3;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + c.wave * S * 32;
    const uint32_t stage = (uint32_t)(size_t)(lds + L.stage + c.wave * STAGE_BYTES);
    const uint32_t my_row = stage + (uint32_t)(c.lane * STAGE_STRIDE);
    // MFMA fragment coordinates of this lane
    const int fr = c.lane & 15, fk = c.lane >> 4;

    // issue every load, tile offsets first; table barrier; own tile (as in fused_q.hip)
    const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
    const LwTabRegs tr = lw_tab_fetch<lw_compact<PLAN>()>(a, false);
    const uint32_t split = a.split[(size_t)c.t * 32 + c.l];
    LwTileRegs64 tile;
    lw_tile_fetch64(a.words, w0, (w1 - w0) >> 5, c.lane, tile);
    lw_tab_put<lw_compact<PLAN>()>(lds, tr, a);
    __syncthreads();                      // the decoder table is complete
    lw_tile_put64(slots, a.words, w0, (w1 - w0) >> 5, c.lane, tile);

    // x fragments: lane holds x[b = fr][col0 + 16 kk + 4 fk .. +3] for kk = 0, 1
    const bool xb_ok = fr < a.batch;
    const uint16_t *xrow = a.x + (size_t)(xb_ok ? fr : 0) * a.cols + (size_t)(c.active ? c.cb : 0) * 256 + 4 * fk;
    auto load_x = [&](int chunk, u32x2 (&dst)[2]) {
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
            const u32x2 v = *reinterpret_cast<const u32x2 *>(xrow + 32 * chunk + 16 * kk);
            dst[kk] = xb_ok ? v : u32x2{0u, 0u};
        }
    };

    f4 acc[4];
#pragma unroll
    for (int r = 0; r < 4; r++) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
    float sx = 0.f;                          // sum of x[fr][k] over this lane's k subset

    if (c.active) {
        LaneDec d;
        const bool ok = lw_lane_init(d, lds, slots, c.l, a);
        d.advance(c.half ? split : 0u);       // the second tile row starts at the split bit
        if (ok) {
            u32x2 xcur[2];
            load_x(0, xcur);
            uint32_t pend = 0;
            auto mfma_step = [&](int chunk) {
#pragma unroll
                for (int kk = 0; kk < 2; kk++) {
                    if constexpr (KIND == LW_BF16_EXP)
                        sx += __builtin_bit_cast(float, xcur[kk].x << 16) +
                              __builtin_bit_cast(float, xcur[kk].x & 0xFFFF0000u) +
                              __builtin_bit_cast(float, xcur[kk].y << 16) +
                              __builtin_bit_cast(float, xcur[kk].y & 0xFFFF0000u);
                    else
                        sx += lw_half_lo(xcur[kk].x) + lw_half_hi(xcur[kk].x) + lw_half_lo(xcur[kk].y) +
                              lw_half_hi(xcur[kk].y);
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const u32x2 af = lw_ld64(stage + (uint32_t)((16 * r + fr) * STAGE_STRIDE + 32 * kk + 8 * fk));
                        acc[r] = mfma<KIND>(af, xcur[kk], acc[r]);
                    }
                }
                // x of the next chunk, used one chunk of decoding later
                load_x(chunk + 1 < 8 ? chunk + 1 : chunk, xcur);
            };
            auto put = [&](int g, int j, uint32_t pay, uint32_t smw) {
                // 16-bit weights of this symbol into the staged row
                if constexpr (KIND == LW_Q4_PAIR) {
                    lw_st32(my_row + (uint32_t)(((g % GPC) * 4 + j) * 4), pay);
                } else {
                    if (j & 1) {
                        uint32_t w2;
                        if constexpr (KIND == LW_BF16_EXP) {
                            const uint32_t spread = __builtin_amdgcn_perm(smw, smw, j == 1 ? 0x01010000u : 0x03030202u);
                            w2 = (spread & 0x807F807Fu) | pend | pay;
                        } else {
                            w2 = pend | pay;
                        }
                        lw_st32(my_row + (uint32_t)(((g % GPC) * 2 + (j >> 1)) * 4), w2);
                    } else {
                        pend = pay;
                    }
                }
                if (j == 3 && (g % GPC) == GPC - 1) mfma_step(g / GPC);
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
            red[(c.wave * NB + fr) * 64 + trow] = v;
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
                    if (c.lane == 0) red[(c.wave * NB + b) * 64 + row] += sb;
                }
            });
        }
        __syncthreads();
    }
    uint32_t *last_flag = reinterpret_cast<uint32_t *>(lds + L.flag);
    lw_finish_rows<NB, 64>(a, red, (int64_t)c.rb * 64, c.g, c.rb, WAVES, last_flag);
}

template <int KIND, int PLAN>
hipError_t launch(const KArgs &a, hipStream_t s)
{
    const LdsLayout L = lds_layout(a.max_words);
    dim3 grid((unsigned)a.groups, (unsigned)a.n_rb);
    auto kern = k_gemv_mfma<KIND, PLAN>;
    hipError_t e = lw_allow_lds<k_gemv_mfma<KIND, PLAN>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(256), L.total, s, a);
    return hipGetLastError();
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
