// skip.hip -- tile-skipping fixed-width GEMV over a launch list of active
// tiles ("Software-Defined Bandwidth Expansion", IV-A storage: 32/b b-bit
// codes per 32-bit word with a scale and zero per group, b in {2, 4, 8};
// IV-B layout: words tile-transposed as [tile][word column][B_N = 64 rows];
// IV-C kernel: one program per active tile does load, unpack in registers,
// scale and zero, and the product with x in one pass, and a skipped tile is
// absent from the grid, so it moves no weight bytes).
//
// Work split.  Each list entry gets two workgroups, one per 32-row half of
// its tile, of 8 * JT threads.  Thread (rq, jl) = (tid % 8, tid / 8) owns
// rows 4rq .. 4rq+3 of the half and the chunks jl, jl + JT, ... of eight
// consecutive word columns; for a fixed word column the half's 32 words are
// contiguous, so one 16-byte load per lane brings four rows' words and the 8
// lanes of a word column read one whole 128-byte line.  A chunk's columns
// lie inside one 256-column group, so one 16-byte load of scales serves it.
//
// Activations.  Each workgroup stages x in LDS once, already arranged as the
// half2 pairs the unpack produces (below), and the sum of x over each chunk
// for the zero term: y_r = sum over chunks of d * sum(q x) - m * sum(x).
//
// Unpack without conversion instructions.
//  b = 4: nibbles i and i+4 of a word moved to bits 6..9 of the two 16-bit
//         halves and masked form the fp16 subnormal pair q * 2^-18, exact;
//  b = 2: crumbs i and i+8 moved to bits 8..9 form q * 2^-16;
//  b = 8: bytes 0 and 2 (1 and 3) under the exponent byte 0x64 form the fp16
//         pair 1024 + q, exact; the 1024 * sum(x) it adds is taken off.
// v_dot2c_f32_f16 takes each pair against the matching x pair.
#include "lane_decode.hpp"

namespace {

constexpr int SK_BN = 64;      // rows per tile (B_N)
constexpr int SK_CW = 8;       // word columns per chunk

template <int BITS>
struct SkipGeom {
    static constexpr int PER = 32 / BITS;            // codes per word
    static constexpr int CC = SK_CW * PER;           // columns per chunk
    static constexpr int XU = PER / 2;               // x pairs per word
    // dwords per chunk of staged pairs: the chunk's 8 words plus 4 of padding,
    // so the 8 chunks a wavefront reads at once start 4 banks apart
    static constexpr int XCS = SK_CW * XU + 4;
};

struct SkipArgs {
    const uint32_t *words;
    const uint32_t *dm;
    const int32_t *tiles;
    const uint16_t *x;
    float *y;
    int64_t rows, cols;
    int32_t n_tiles, n_jc, jt;
};

constexpr int SK_RW = 32;      // rows per workgroup (half a tile)

struct SkipLds {
    uint32_t xs, sxs, total;
};

// LDS: the staged x pairs (later reused for the per-wave partial rows),
// then the per-chunk sums of x.
__host__ __device__ inline SkipLds skip_lds(int batch, int64_t cols, int n_jc, int jt)
{
    SkipLds L;
    const uint32_t xbytes = (uint32_t)(batch * cols * 2 + batch * n_jc * 16);
    const uint32_t red = (uint32_t)((jt / 8) * batch * SK_RW * 4);
    L.xs = 0;
    L.sxs = xbytes > red ? xbytes : red;
    L.total = L.sxs + (uint32_t)(batch * n_jc * 4);
    return L;
}

// half2 pairs of one word's PER activations in unpack order: pair i is
// (x_i, x_{i+PER/2}); X holds the PER halves as PER/2 dwords
template <int BITS>
LW_DEV void arrange_pairs(const uint32_t *X, uint32_t *out)
{
    constexpr int H = SkipGeom<BITS>::XU;            // dwords per half of the word's activations
#pragma unroll
    for (int i = 0; i < H; i++)
        out[i] = __builtin_amdgcn_perm(X[H / 2 + i / 2], X[i / 2], (i & 1) ? 0x07060302u : 0x05040100u);
}

// sum over one word's four unpacked pair sets of dot(pair, x pair), for one row
template <int BITS>
LW_DEV float word_dot(uint32_t w, const uint32_t *xp, float s)
{
    if constexpr (BITS == 4) {
        const uint32_t M = 0x03C003C0u;
        s = lw_dot2((w << 6) & M, xp[0], s);
        s = lw_dot2((w << 2) & M, xp[1], s);
        s = lw_dot2((w >> 2) & M, xp[2], s);
        s = lw_dot2((w >> 6) & M, xp[3], s);
    } else if constexpr (BITS == 2) {
        const uint32_t M = 0x03000300u;
        s = lw_dot2((w << 8) & M, xp[0], s);
        s = lw_dot2((w << 6) & M, xp[1], s);
        s = lw_dot2((w << 4) & M, xp[2], s);
        s = lw_dot2((w << 2) & M, xp[3], s);
        s = lw_dot2(w & M, xp[4], s);
        s = lw_dot2((w >> 2) & M, xp[5], s);
        s = lw_dot2((w >> 4) & M, xp[6], s);
        s = lw_dot2((w >> 6) & M, xp[7], s);
    } else {
        s = lw_dot2(__builtin_amdgcn_perm(0x64646464u, w, 0x04020400u), xp[0], s);
        s = lw_dot2(__builtin_amdgcn_perm(0x64646464u, w, 0x04030401u), xp[1], s);
    }
    return s;
}

// word_dot's unpacked code is q * 2^-18 (b = 4), q * 2^-16 (b = 2) or
// 1024 + q (b = 8): the factor that turns its sum back into sum(q x)
template <int BITS>
constexpr float unpack_scale()
{
    return BITS == 4 ? 262144.0f : BITS == 2 ? 65536.0f : 1.0f;
}

struct Chunk {
    lw_u32x4 w[SK_CW];       // word column i, rows 4rq .. 4rq+3
    lw_u32x4 dm;             // (d, m) of the four rows for the chunk's group
};

// r0: the first of the lane's four rows within the tile
LW_DEV void load_chunk(const SkipArgs &a, int t, int jc, int r0, int cc, Chunk &c)
{
    const int64_t wpr = (int64_t)a.n_jc * SK_CW;
    const lw_u32x4 *src =
        reinterpret_cast<const lw_u32x4 *>(a.words + ((int64_t)t * wpr + (int64_t)jc * SK_CW) * SK_BN + r0);
#pragma unroll
    for (int i = 0; i < SK_CW; i++) c.w[i] = src[i * (SK_BN / 4)];
    const int64_t ng = a.cols / 256;
    const int64_t g = (int64_t)jc * cc / 256;
    c.dm = *reinterpret_cast<const lw_u32x4 *>(a.dm + ((int64_t)t * ng + g) * SK_BN + r0);
}

template <int BITS, int BATCH>
__global__ __launch_bounds__(1024) void k_skip(SkipArgs a)
{
    using G = SkipGeom<BITS>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = a.tiles[blockIdx.x >> 1];
    if (t < 0 || t >= a.n_tiles) return;                 // names no tile: the whole workgroup leaves
    const int half = blockIdx.x & 1;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int rq = tid & 7, jl = tid >> 3;
    const int r0 = half * SK_RW + 4 * rq;                // the lane's first row within the tile
    const int n_jc = a.n_jc, JT = a.jt;
    const int n_it = (n_jc + JT - 1) / JT;
    const SkipLds L = skip_lds(BATCH, a.cols, n_jc, JT);
    const uint32_t lb = (uint32_t)(size_t)lds;

    // the first chunk's words and scales are in flight while x is staged
    Chunk c;
    load_chunk(a, t, min(jl, n_jc - 1), r0, G::CC, c);

    // stage x: item (b, j) arranges word column j's activations of batch row
    // b; the 8 items of a chunk sit in 8 aligned consecutive lanes, which sum
    // the chunk's activations by lane sums (the item count is a multiple of 8)
    const int wpc = a.n_jc * SK_CW;                      // word columns of the matrix
    for (int item = tid; item < BATCH * wpc; item += nt) {
        const int b = item / wpc, j = item % wpc;
        const uint32_t *xg = reinterpret_cast<const uint32_t *>(a.x + (int64_t)b * a.cols) + (int64_t)j * G::XU;
        uint32_t X[G::XU], P[G::XU];
        if constexpr (G::XU == 2) {
            const uint2 v = *reinterpret_cast<const uint2 *>(xg);
            X[0] = v.x; X[1] = v.y;
        } else {
#pragma unroll
            for (int k = 0; k < G::XU; k += 4) {
                const uint4 v = *reinterpret_cast<const uint4 *>(xg + k);
                X[k] = v.x; X[k + 1] = v.y; X[k + 2] = v.z; X[k + 3] = v.w;
            }
        }
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < G::XU; k++) s = lw_dot2(X[k], 0x3C003C00u, s);          // times half2(1, 1)
        arrange_pairs<BITS>(X, P);
        const uint32_t ad = lb + L.xs + 4u * (uint32_t)((b * n_jc + j / SK_CW) * G::XCS + (j % SK_CW) * G::XU);
#pragma unroll
        for (int k = 0; k < G::XU; k++) *(lw_lds_w32 *)(size_t)(ad + 4u * k) = P[k];
        s = lw_group_sum<8>(s);                          // whole 8-lane groups are active
        if ((j & 7) == 0)
            *(lw_lds_w32 *)(size_t)(lb + L.sxs + 4u * (uint32_t)(b * n_jc + j / SK_CW)) = __builtin_bit_cast(uint32_t, s);
    }
    __syncthreads();

    float acc[4][BATCH];
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
        for (int b = 0; b < BATCH; b++) acc[r][b] = 0.f;

    auto compute = [&](int jc) {
        float s[4][BATCH];
#pragma unroll
        for (int r = 0; r < 4; r++)
#pragma unroll
            for (int b = 0; b < BATCH; b++) s[r][b] = 0.f;
#pragma unroll
        for (int i = 0; i < SK_CW; i++) {
#pragma unroll
            for (int b = 0; b < BATCH; b++) {
                uint32_t xp[G::XU];
                const uint32_t ad = lb + L.xs + 4u * (uint32_t)((b * n_jc + jc) * G::XCS + i * G::XU);
                if constexpr (G::XU == 8) {
                    const lw_u32x4 u = *(__attribute__((address_space(3))) const lw_u32x4 *)(size_t)ad;
                    const lw_u32x4 v = *(__attribute__((address_space(3))) const lw_u32x4 *)(size_t)(ad + 16);
                    xp[0] = u.x; xp[1] = u.y; xp[2] = u.z; xp[3] = u.w;
                    xp[4] = v.x; xp[5] = v.y; xp[6] = v.z; xp[7] = v.w;
                } else if constexpr (G::XU == 4) {
                    const lw_u32x4 u = *(__attribute__((address_space(3))) const lw_u32x4 *)(size_t)ad;
                    xp[0] = u.x; xp[1] = u.y; xp[2] = u.z; xp[3] = u.w;
                } else {
                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                    const u32x2 u = *(__attribute__((address_space(3))) const u32x2 *)(size_t)ad;
                    xp[0] = u.x; xp[1] = u.y;
                }
                s[0][b] = word_dot<BITS>(c.w[i].x, xp, s[0][b]);
                s[1][b] = word_dot<BITS>(c.w[i].y, xp, s[1][b]);
                s[2][b] = word_dot<BITS>(c.w[i].z, xp, s[2][b]);
                s[3][b] = word_dot<BITS>(c.w[i].w, xp, s[3][b]);
            }
        }
        const uint32_t dmr[4] = {c.dm.x, c.dm.y, c.dm.z, c.dm.w};
#pragma unroll
        for (int b = 0; b < BATCH; b++) {
            const float sx = __builtin_bit_cast(float, *(lw_lds_u32 *)(size_t)(lb + L.sxs + 4u * (uint32_t)(b * n_jc + jc)));
#pragma unroll
            for (int r = 0; r < 4; r++) {
                float sq = s[r][b] * unpack_scale<BITS>();
                if constexpr (BITS == 8) sq -= 1024.0f * sx;
                acc[r][b] += lw_half_lo(dmr[r]) * sq - lw_half_hi(dmr[r]) * sx;
            }
        }
    };

    // one chunk in registers at a time (a second buffer would spill at batch > 1);
    // the other workgroups' waves on the compute unit cover the reload latency
    for (int it = 0; it < n_it; it++) {
        const int jc = jl + it * JT;
        if (it > 0) load_chunk(a, t, min(jc, n_jc - 1), r0, G::CC, c);
        if (jc < n_jc) compute(jc);
    }

    // rows: sum over the wave's eight chunk lanes, then over the waves in LDS
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
        for (int b = 0; b < BATCH; b++) {
            float v = acc[r][b];
            v = lw_dpp_add<0x128>(v);                   // row_ror:8, lane i ^ 8 within its row
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[r][b] = v;
        }
    __syncthreads();                                      // x no longer read: its space holds the partials
    const int wave = tid >> 6, lane = tid & 63;
    float *red = reinterpret_cast<float *>(lds + L.xs);
    if (lane < 8) {
#pragma unroll
        for (int r = 0; r < 4; r++)
#pragma unroll
            for (int b = 0; b < BATCH; b++) red[(wave * BATCH + b) * SK_RW + 4 * rq + r] = acc[r][b];
    }
    __syncthreads();
    const int waves = nt >> 6;
    for (int i = tid; i < BATCH * SK_RW; i += nt) {
        const int b = i / SK_RW, row = i % SK_RW;
        float v = 0.f;
        for (int w = 0; w < waves; w++) v += red[(w * BATCH + b) * SK_RW + row];
        a.y[(int64_t)b * a.rows + (int64_t)t * SK_BN + half * SK_RW + row] = v;
    }
}

template <int BITS, int BATCH>
hipError_t launch_skip(const SkipArgs &a, int64_t n_list, hipStream_t s)
{
    const SkipLds L = skip_lds(BATCH, a.cols, a.n_jc, a.jt);
    if (L.total > (uint32_t)lw_device_lds_bytes()) return hipErrorNotSupported;
    hipError_t e = lw_allow_lds<k_skip<BITS, BATCH>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_skip<BITS, BATCH>), dim3((unsigned)(2 * n_list)), dim3(8 * a.jt), L.total, s, a);
    return hipGetLastError();
}

template <int BITS>
hipError_t skip_batch(const SkipArgs &a, int64_t n_list, int batch, hipStream_t s)
{
    switch (batch) {
    case 1: return launch_skip<BITS, 1>(a, n_list, s);
    case 2: return launch_skip<BITS, 2>(a, n_list, s);
    case 3: return launch_skip<BITS, 3>(a, n_list, s);
    case 4: return launch_skip<BITS, 4>(a, n_list, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t lw_launch_skip(const uint32_t *words, const uint32_t *dm, int bits, int64_t rows, int64_t cols,
                          const int32_t *tiles, int64_t n_list, const uint16_t *x, float *y, int batch,
                          hipStream_t s)
{
    SkipArgs a;
    a.words = words;
    a.dm = dm;
    a.tiles = tiles;
    a.x = x;
    a.y = y;
    a.rows = rows;
    a.cols = cols;
    a.n_tiles = (int32_t)(rows / SK_BN);
    const int cc = SK_CW * (32 / bits);
    a.n_jc = (int32_t)(cols / cc);
    const int jt = a.n_jc < 128 ? ((a.n_jc + 7) / 8) * 8 : 128;   // chunk lanes: whole wavefronts, at most 16 waves
    a.jt = jt;
    switch (bits) {
    case 2: return skip_batch<2>(a, n_list, batch, s);
    case 4: return skip_batch<4>(a, n_list, batch, s);
    case 8: return skip_batch<8>(a, n_list, batch, s);
    }
    return hipErrorInvalidValue;
}
