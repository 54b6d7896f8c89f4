// twin.hip -- GEMV over the fixed-width 4-bit "twin" (the decode-free
// stand-in of the runtime paragraph under "LazyWeights" Fig. 3; grouped
// packing of "Software-Defined Bandwidth Expansion" IV-A/IV-C: load packed
// words, unpack in registers, apply scale and zero, accumulate with x).
//
// Layout: codes [rows][cols/2] bytes, low nibble = even column; dm
// [rows][cols/256] u32 = d | m << 16.  A workgroup of 256 threads handles
// RG row groups of R rows; the TPR threads of a row group stride over the
// row's 32-column chunks (16 bytes of codes per row per chunk, one 16-byte
// load per row), so every load is a fully used, aligned 16-byte access and
// one x chunk serves R rows.  Nibbles become fp16 exactly through the
// 0x6400 exponent trick (half(1024 + q) - 1024), then v_dot2_f32_f16.
#include "kernels.h"
#include "lane_decode.hpp"

namespace {

// eight nibbles of w (columns 0..7 of a chunk word) as four half2 pairs
// (q0,q4) (q1,q5) (q2,q6) (q3,q7)
LW_DEV void unpack8(uint32_t w, uint32_t out[4])
{
    const uint32_t magic = 0x64006400u;
    const lw_half2 bias = {(_Float16)-1024.0f, (_Float16)-1024.0f};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t v = ((w >> (4 * i)) & 0x000F000Fu) | magic;
        lw_half2 h = __builtin_bit_cast(lw_half2, v) + bias;
        out[i] = __builtin_bit_cast(uint32_t, h);
    }
}

// x pairs matching unpack8: from 8 halves (x0..x7 in dwords X0..X3) form
// (x0,x4) (x1,x5) (x2,x6) (x3,x7)
LW_DEV void xpairs8(uint32_t X0, uint32_t X1, uint32_t X2, uint32_t X3, uint32_t out[4])
{
    out[0] = __builtin_amdgcn_perm(X2, X0, 0x05040100u);   // (x0, x4)
    out[1] = __builtin_amdgcn_perm(X2, X0, 0x07060302u);   // (x1, x5)
    out[2] = __builtin_amdgcn_perm(X3, X1, 0x05040100u);   // (x2, x6)
    out[3] = __builtin_amdgcn_perm(X3, X1, 0x07060302u);   // (x3, x7)
}

template <int TPR, int R, int BATCH>
__global__ __launch_bounds__(256) void k_twin(const uint8_t *__restrict__ twin, const uint32_t *__restrict__ dm,
                                              int64_t rows, int64_t cols, const uint16_t *__restrict__ x,
                                              float *__restrict__ y)
{
    constexpr int RG = 256 / TPR;
    const int rg = threadIdx.x / TPR, t = threadIdx.x % TPR;
    const int64_t row0 = ((int64_t)blockIdx.x * RG + rg) * R;
    const int64_t nchunk = cols / 32, nsb = cols / 256;
    float acc[R][BATCH];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int b = 0; b < BATCH; b++) acc[r][b] = 0.f;

    for (int64_t ch = t; ch < nchunk; ch += TPR) {
        uint4 q[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int64_t row = row0 + r < rows ? row0 + r : rows - 1;
            q[r] = *reinterpret_cast<const uint4 *>(twin + row * (cols / 2) + ch * 16);
        }
        float d[R], m[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int64_t row = row0 + r < rows ? row0 + r : rows - 1;
            const uint32_t v = dm[row * nsb + ch / 8];
            d[r] = lw_half_lo(v);
            m[r] = lw_half_hi(v);
        }
#pragma unroll
        for (int b = 0; b < BATCH; b++) {
            const uint4 *xc = reinterpret_cast<const uint4 *>(x + (int64_t)b * cols + ch * 32);
            uint32_t xp[4][4];
            float sx = 0.f;
#pragma unroll
            for (int j = 0; j < 4; j++) {        // 8 columns per j
                const uint4 X = xc[j];
                xpairs8(X.x, X.y, X.z, X.w, xp[j]);
                sx += lw_half_lo(X.x) + lw_half_hi(X.x) + lw_half_lo(X.y) + lw_half_hi(X.y) +
                      lw_half_lo(X.z) + lw_half_hi(X.z) + lw_half_lo(X.w) + lw_half_hi(X.w);
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                const uint32_t w4[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    uint32_t qp[4];
                    unpack8(w4[j], qp);
#pragma unroll
                    for (int i = 0; i < 4; i++) s = lw_dot2(qp[i], xp[j][i], s);
                }
                acc[r][b] += d[r] * s - m[r] * sx;
            }
        }
    }
    // reduce over the TPR threads of the row group
    __shared__ float red[256 / 64][R * BATCH];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int b = 0; b < BATCH; b++) {
            float v = acc[r][b];
#pragma unroll
            for (int o = (TPR < 64 ? TPR : 64) / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
            acc[r][b] = v;
        }
    if (TPR <= 64) {
        if (t == 0) {
#pragma unroll
            for (int r = 0; r < R; r++)
                if (row0 + r < rows)
#pragma unroll
                    for (int b = 0; b < BATCH; b++) y[(int64_t)b * rows + row0 + r] = acc[r][b];
        }
        return;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int b = 0; b < BATCH; b++) red[wave][r * BATCH + b] = acc[r][b];
    }
    __syncthreads();
    constexpr int WPR = TPR / 64;               // waves per row group
    if (t < R * BATCH) {
        const int r = t / BATCH, b = t % BATCH;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < WPR; w++) v += red[rg * WPR + w][r * BATCH + b];
        if (row0 + r < rows) y[(int64_t)b * rows + row0 + r] = v;
    }
}

template <int TPR, int R, int BATCH>
hipError_t launch(const uint8_t *twin, const uint32_t *dm, int64_t rows, int64_t cols, const uint16_t *x,
                  float *y, hipStream_t s)
{
    constexpr int RG = 256 / TPR;
    const int64_t per_block = (int64_t)RG * R;
    dim3 grid((unsigned)((rows + per_block - 1) / per_block));
    hipLaunchKernelGGL((k_twin<TPR, R, BATCH>), grid, dim3(256), 0, s, twin, dm, rows, cols, x, y);
    return hipGetLastError();
}

template <int BATCH>
hipError_t by_shape(const uint8_t *twin, const uint32_t *dm, int64_t rows, int64_t cols, const uint16_t *x,
                    float *y, hipStream_t s)
{
    const int64_t nchunk = cols / 32;
    if (nchunk >= 256) return launch<256, 4, BATCH>(twin, dm, rows, cols, x, y, s);
    if (nchunk >= 128) return launch<128, 4, BATCH>(twin, dm, rows, cols, x, y, s);
    if (nchunk >= 64) return launch<64, 4, BATCH>(twin, dm, rows, cols, x, y, s);
    return launch<32, 4, BATCH>(twin, dm, rows, cols, x, y, s);
}

}  // namespace

hipError_t lw_launch_twin(const uint8_t *twin, const uint32_t *dm, int64_t rows, int64_t cols,
                          const uint16_t *x, float *y, int batch, hipStream_t s)
{
    switch (batch) {
    case 1: return by_shape<1>(twin, dm, rows, cols, x, y, s);
    case 2: return by_shape<2>(twin, dm, rows, cols, x, y, s);
    case 3: return by_shape<3>(twin, dm, rows, cols, x, y, s);
    case 4: return by_shape<4>(twin, dm, rows, cols, x, y, s);
    case 5: return by_shape<5>(twin, dm, rows, cols, x, y, s);
    case 6: return by_shape<6>(twin, dm, rows, cols, x, y, s);
    case 7: return by_shape<7>(twin, dm, rows, cols, x, y, s);
    case 8: return by_shape<8>(twin, dm, rows, cols, x, y, s);
    case 9: return by_shape<9>(twin, dm, rows, cols, x, y, s);
    case 10: return by_shape<10>(twin, dm, rows, cols, x, y, s);
    case 11: return by_shape<11>(twin, dm, rows, cols, x, y, s);
    case 12: return by_shape<12>(twin, dm, rows, cols, x, y, s);
    case 13: return by_shape<13>(twin, dm, rows, cols, x, y, s);
    case 14: return by_shape<14>(twin, dm, rows, cols, x, y, s);
    case 15: return by_shape<15>(twin, dm, rows, cols, x, y, s);
    case 16: return by_shape<16>(twin, dm, rows, cols, x, y, s);
    }
    return hipErrorInvalidValue;
}
