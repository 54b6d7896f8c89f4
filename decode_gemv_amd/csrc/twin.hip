// twin.hip -- GEMV over the fixed-width 4-bit "twin" (the decode-free
// stand-in of the runtime paragraph under "LazyWeights" Fig. 3; grouped
// packing of "Software-Defined Bandwidth Expansion" IV-A/IV-C: load packed
// words, unpack in registers, apply scale and zero, accumulate with x).
//
// Layout: codes [rows][cols/2] bytes, low nibble = even column; dm
// [rows][cols/256] u32 = d | m << 16.  A workgroup of 256 threads handles
// RG row groups of R rows; the TPR threads of a row group stride over the
// row's 32-column chunks (16 bytes of codes per row per chunk), two chunks
// per step with all loads issued first, so every load is a fully used,
// aligned 16-byte access and one x chunk serves R rows.
//
// Unpacking needs no conversion: a nibble moved to bits 6..9 of each 16-bit
// half and masked with 0x03C003C0 is the fp16 subnormal q * 2^-18, exact, so
// v_dot2c_f32_f16 takes it straight against the matching x pair and the chunk
// sum is rescaled once by 2^18.  Bits 6..9 and no lower: the dot unit aligns
// its addends to the exponent a subnormal operand would have if normal
// (2^-14), and an accumulating chain of dot2s whose subnormal operand sits k
// bits below that loses about k bits of the running sum (measured on gfx950:
// nibbles at bits 0..3 cost six bits, at bits 6..9 none against a plain fp32
// sum).  Per eight weights: four shifts, four ANDs and four dot products, all
// 4-byte VOP2 encodings.
#include "lane_decode.hpp"

namespace {

// x pairs matching the nibble order: from 8 halves (x0..x7 in dwords X0..X3)
// form (x0,x4) (x1,x5) (x2,x6) (x3,x7)
LW_DEV void xpairs8(uint32_t X0, uint32_t X1, uint32_t X2, uint32_t X3, uint32_t out[4])
{
    out[0] = __builtin_amdgcn_perm(X2, X0, 0x05040100u);   // (x0, x4)
    out[1] = __builtin_amdgcn_perm(X2, X0, 0x07060302u);   // (x1, x5)
    out[2] = __builtin_amdgcn_perm(X3, X1, 0x05040100u);   // (x2, x6)
    out[3] = __builtin_amdgcn_perm(X3, X1, 0x07060302u);   // (x3, x7)
}

struct XChunk {
    uint32_t p[4][4];                     // [word j][pair]
    float sx;                             // sum of the chunk's 32 x values
};

LW_DEV XChunk load_x(const uint16_t *x, int64_t ch)
{
    XChunk c;
    const uint4 *xc = reinterpret_cast<const uint4 *>(x + ch * 32);
    float s = 0.f;
    const uint32_t ones = 0x3C003C00u;                     // half2(1, 1)
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint4 X = xc[j];
        xpairs8(X.x, X.y, X.z, X.w, c.p[j]);
        s = lw_dot2(X.x, ones, s);
        s = lw_dot2(X.y, ones, s);
        s = lw_dot2(X.z, ones, s);
        s = lw_dot2(X.w, ones, s);
    }
    c.sx = s;
    return c;
}

// sum(q x) * 2^-18 over a 16-byte chunk of codes; nibble i of a word (bits
// 4i..4i+3, partner 4i+16..) is shifted by 6 - 4i to reach bits 6..9
LW_DEV float chunk_dot(const uint4 &q, const XChunk &xc)
{
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
    const uint32_t mask = 0x03C003C0u;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t w = w4[j];
        a = lw_dot2((w << 6) & mask, xc.p[j][0], a);
        b = lw_dot2((w << 2) & mask, xc.p[j][1], b);
        a = lw_dot2((w >> 2) & mask, xc.p[j][2], a);
        b = lw_dot2((w >> 6) & mask, xc.p[j][3], b);
    }
    return a + b;
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
    int64_t rowc[R];
#pragma unroll
    for (int r = 0; r < R; r++) rowc[r] = row0 + r < rows ? row0 + r : rows - 1;

    for (int64_t ch0 = t; ch0 < nchunk; ch0 += 2 * TPR) {
        const int64_t ch1 = ch0 + TPR < nchunk ? ch0 + TPR : ch0;
        const bool two = ch0 + TPR < nchunk;
        uint4 q[2][R];
        uint32_t dmv[2][R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            q[0][r] = *reinterpret_cast<const uint4 *>(twin + rowc[r] * (cols / 2) + ch0 * 16);
            q[1][r] = *reinterpret_cast<const uint4 *>(twin + rowc[r] * (cols / 2) + ch1 * 16);
            dmv[0][r] = dm[rowc[r] * nsb + ch0 / 8];
            dmv[1][r] = dm[rowc[r] * nsb + ch1 / 8];
        }
#pragma unroll
        for (int b = 0; b < BATCH; b++) {
#pragma unroll
            for (int u = 0; u < 2; u++) {
                if (u == 1 && !two) break;
                const XChunk xc = load_x(x + (int64_t)b * cols, u ? ch1 : ch0);
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const float sqx = chunk_dot(q[u][r], xc) * 262144.0f;
                    acc[r][b] += lw_half_lo(dmv[u][r]) * sqx - lw_half_hi(dmv[u][r]) * xc.sx;
                }
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

// threads per row: enough 32-column chunks for two per thread where possible
template <int BATCH>
hipError_t by_shape(const uint8_t *twin, const uint32_t *dm, int64_t rows, int64_t cols, const uint16_t *x,
                    float *y, hipStream_t s)
{
    const int64_t nchunk = cols / 32;
    if (nchunk >= 512) return launch<256, 4, BATCH>(twin, dm, rows, cols, x, y, s);
    if (nchunk >= 256) return launch<128, 4, BATCH>(twin, dm, rows, cols, x, y, s);
    if (nchunk >= 128) return launch<64, 4, BATCH>(twin, dm, rows, cols, x, y, s);
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
