// recon.hip -- reconstructive matrix-core GEMM for bf16 bundles ("Unweight:
// Compressing LLM Weights for Faster Inference", sections "Four approaches to
// using compressed weights" and "How reconstructive matmul works"): the
// weights are rebuilt in registers from a compact form and fed straight to
// the matrix cores; they never exist in memory as bf16.
//
//   y[b][r] = sum_c W[r][c] x[b][c],   W[r][c] = bf16(sign+mantissa byte, exponent)
//
// The exponent comes from a 4-bit palette index (SRC_PALETTE: the runtime
// palette transcode and the direct-palette pipelines) or from an exponent
// byte (SRC_EXPONENT: the exponent-only pipeline), both written by the
// transcode kernel in a tile-major layout; the sign+mantissa byte comes from
// the bundle itself; a 64-weight segment stored verbatim replaces the rebuilt
// weights by its stored values, found through the transcode's rank table.
//
// MI355X mapping.  v_mfma_f32_16x16x32_bf16 computes a 16x16 block of y^T
// (16 weight rows by 16 batch columns) over 32 columns: lane l holds weights
// W[r0 + l%16][k0 + 8(l/16) .. + 7] (A), activations x[b0 + l%16][same
// columns] (B) and y^T rows r0 + 4(l/16) .. + 3 of column b0 + l%16 (D).
// A workgroup is four wavefronts on 64 weight rows (one row band of the
// bundle).  Either each wavefront owns 16 of the rows and all the
// workgroup's batch columns, keeping its rebuilt operand in registers, or
// (large batches) each rebuilds its 16 rows into an LDS tile and multiplies
// all 64 rows with its own quarter of the batch columns, so one rebuilt
// operand feeds four times as many matrix instructions.  The activations of
// a 32-column step are shared through an LDS double buffer (16-byte chunks
// swizzled within a row, so stores and B reads are free of bank conflicts).
//
// Rebuilding eight weights (one A operand) from the palette form: the eight
// indices give eight bytes T = ror8(exponent) by two byte permutes over the
// palette (indices 0-7 and 8-15) and a mask; a pair of weights is then
//   bfi(0x807F807F, [s0 s0 s1 s1], [t0 t0 t1 t1])
// (sign and mantissa from the sm byte, exponent from T: the high byte takes
// T's bits 6..0 as exponent bits 7..1 and the sm sign, the low byte T's bit 7
// as exponent bit 0 and the sm mantissa).  About 3.6 VALU instructions a
// weight; the exponent form needs about 2.3.
//
// Latency.  The weight sources (compact form, sm words, verbatim rank) of
// step k + 3 are requested during step k (a ring of four), and the
// activations of step k + 1, stored to the other LDS buffer at the step's
// end; one barrier per step.  A workgroup's verbatim segments are one run of
// the store (it is ordered by tile, row and segment): the run is staged in
// LDS at the start when it holds at most VCAP segments, so a rebuilt operand
// that falls in one reads its stored values from LDS.
#include <type_traits>

#include "lane_decode.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int XSTRIDE = 64;                  // bytes per staged activation row (32 bf16)

// 16-byte chunk q of staged row r sits at chunk q ^ ((r >> 2) & 3): the 16
// lanes of a B read (rows r0 .. r0+15, one chunk) and the 16 lanes of a
// store (rows r0 .. r0+3, all four chunks) then hit 16 distinct groups of
// four banks
__device__ __forceinline__ int xs_off(int r, int q) { return r * XSTRIDE + 16 * (q ^ ((r >> 2) & 3)); }

struct RArgs {
    const uint32_t *src;        // palette: [t][32][64] u32 (8 indices); exponent: [t][64][64] u32 (4 bytes)
    const uint32_t *sm;         // bundle sign+mantissa words [t][2][64][32]
    const int32_t *vrank;       // [t][4][64] verbatim store index, or -1
    const uint32_t *vb_start;   // [n_tiles + 1] verbatim segments before each tile
    int64_t n_verbatim;         // segments in the verbatim store
    const uint16_t *verbatim;   // [n][64] stored bf16 segments
    const uint16_t *x;          // [batch][cols] bf16
    float *y;                   // [batch][rows]
    float *part;                // [splits][batch][rows] partial sums when the columns are split
    int splits;                 // column-block ranges, one per blockIdx.z
    int64_t rows, cols;
    int ncb, batch;
    uint32_t t03, t47, t8b, tcf; // palette as T = ror8(exponent) bytes, indices 0-3, 4-7, 8-11, 12-15
};

// Four palette indices (one a byte, 0..15) -> their four T bytes.
LW_DEV uint32_t lw_lookup4(uint32_t idx4, const RArgs &a)
{
    const uint32_t plo = __builtin_amdgcn_perm(a.t47, a.t03, idx4);                    // valid for 0..7
    const uint32_t phi = __builtin_amdgcn_perm(a.tcf, a.t8b, idx4 ^ 0x08080808u);      // valid for 8..15
    const uint32_t msel = ((idx4 >> 3) & 0x01010101u) | 0x0C0C0C0Cu;                  // 0x0C -> 0x00, 0x0D -> 0xFF
    const uint32_t m = __builtin_amdgcn_perm(0u, 0u, msel);
    return (phi & m) | (plo & ~m);
}

template <bool EXP>
LW_DEV u32x4 lw_rebuild8(uint32_t s0, uint32_t s1, uint32_t sm_lo, uint32_t sm_hi, const RArgs &a)
{
    u32x4 w;
    if constexpr (EXP) {
        // s0, s1: exponent bytes of columns 0-3 and 4-7; T = ror8(e)
        const uint32_t tl = (s0 >> 1 & 0x7F7F7F7Fu) | (s0 << 7 & 0x80808080u);
        const uint32_t th = (s1 >> 1 & 0x7F7F7F7Fu) | (s1 << 7 & 0x80808080u);
        w.x = __builtin_amdgcn_perm(tl, tl, 0x01010000u);
        w.y = __builtin_amdgcn_perm(tl, tl, 0x03030202u);
        w.z = __builtin_amdgcn_perm(th, th, 0x01010000u);
        w.w = __builtin_amdgcn_perm(th, th, 0x03030202u);
    } else {
        // s0: eight nibbles; even columns' indices in bytes of ie, odd in io
        const uint32_t te = lw_lookup4(s0 & 0x0F0F0F0Fu, a);
        const uint32_t to = lw_lookup4((s0 >> 4) & 0x0F0F0F0Fu, a);
        w.x = __builtin_amdgcn_perm(to, te, 0x04040000u);
        w.y = __builtin_amdgcn_perm(to, te, 0x05050101u);
        w.z = __builtin_amdgcn_perm(to, te, 0x06060202u);
        w.w = __builtin_amdgcn_perm(to, te, 0x07070303u);
    }
    w.x = __builtin_amdgcn_perm(sm_lo, sm_lo, 0x01010000u) & 0x807F807Fu | (w.x & ~0x807F807Fu);
    w.y = __builtin_amdgcn_perm(sm_lo, sm_lo, 0x03030202u) & 0x807F807Fu | (w.y & ~0x807F807Fu);
    w.z = __builtin_amdgcn_perm(sm_hi, sm_hi, 0x01010000u) & 0x807F807Fu | (w.z & ~0x807F807Fu);
    w.w = __builtin_amdgcn_perm(sm_hi, sm_hi, 0x03030202u) & 0x807F807Fu | (w.w & ~0x807F807Fu);
    return w;
}

constexpr int VCAP = 128;                    // verbatim segments a workgroup stages in LDS

template <bool EXP>
struct Src {
    uint32_t s0, s1, lo, hi;
    int32_t vr;
};

// Modes: MODE 0 splits the workgroup's 64 rows between the wavefronts (each
// keeps its rebuilt operand in registers and covers all 16*NB batch columns);
// MODE 1 splits the batch: each wavefront rebuilds its 16 rows into the LDS
// A tile and covers all 64 rows for its own 16*NB columns (the workgroup's
// batch tile is 64*NB columns), so every rebuilt operand feeds 4*NB matrix
// instructions instead of NB.
template <bool EXP, int MODE, int NB>
__global__ __launch_bounds__(256, 2) void k_recon(RArgs a)
{
    constexpr int BN = MODE ? 64 * NB : 16 * NB;            // batch columns of the workgroup
    constexpr int XV = (BN * 4 + 255) / 256;                 // 16-byte activation chunks per thread and step
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][BN][XSTRIDE];
    __shared__ __attribute__((aligned(16))) u32x4 as[2][MODE ? 4 : 1][64];
    __shared__ __attribute__((aligned(16))) uint16_t vs[VCAP][64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, j = lane & 15;
    const int64_t row0 = (int64_t)blockIdx.x * 64;                      // the workgroup's 64 rows
    const int b0 = blockIdx.y * BN;
    // this workgroup's whole column blocks [cb0, cb1): steps [kbeg, kend)
    const int ncbz = a.ncb, sz = (int)blockIdx.z;
    const int kbeg = 8 * (int)((int64_t)ncbz * sz / a.splits), kend = 8 * (int)((int64_t)ncbz * (sz + 1) / a.splits);

    // The verbatim segments of the workgroup's row band are one run of the
    // store (ordered by tile, tile row, segment), [v0, v1): staged in LDS
    // when the run fits, else read from memory where used.
    const int64_t rb = row0 >> 6;
    const uint32_t v0 = a.vb_start[rb * a.ncb], v1 = a.vb_start[(rb + 1) * a.ncb];
    const bool staged = v1 - v0 <= (uint32_t)VCAP;
    if (staged)
        for (uint32_t i = threadIdx.x; i < (v1 - v0) * 8; i += 256)
            reinterpret_cast<u32x4 *>(&vs[0][0])[i] = reinterpret_cast<const u32x4 *>(a.verbatim + (int64_t)v0 * 64)[i];

    const int64_t t0 = rb * a.ncb;                                       // tile of column block 0
    const uint32_t *srcw = a.src + t0 * (EXP ? 4096 : 2048);
    const uint32_t *smw = a.sm + t0 * 4096;
    const int32_t *vrw = a.vrank + t0 * 256;
    const uint32_t i = (uint32_t)(16 * wave + j);                        // this lane's tile row

    auto src_load = [&](int k, Src<EXP> &s) {
        const uint32_t cb = (uint32_t)(k >> 3), cl = 32u * (k & 7) + 8u * q;
        if constexpr (EXP) {
            s.s0 = srcw[cb * 4096u + (cl >> 2) * 64u + i];
            s.s1 = srcw[cb * 4096u + ((cl >> 2) + 1u) * 64u + i];
        } else {
            s.s0 = srcw[cb * 2048u + (cl >> 3) * 64u + i];
        }
        const uint32_t so = cb * 4096u + (i & 1u) * 2048u + (cl >> 2) * 32u + (i >> 1);
        s.lo = smw[so];
        s.hi = smw[so + 32u];
        s.vr = vrw[cb * 256u + ((k & 7) >> 1) * 64u + i];
    };
    auto x_load = [&](int k, u32x4 (&xr)[XV]) {
#pragma unroll
        for (int m = 0; m < XV; m++) {
            const int id = threadIdx.x + 256 * m;
            const int jj = min(id >> 2, BN - 1), qq = id & 3;
            const int b = min(b0 + jj, a.batch - 1);
            xr[m] = *reinterpret_cast<const u32x4 *>(a.x + (int64_t)b * a.cols + 32 * k + 8 * qq);
        }
    };
    auto x_store = [&](int buf, const u32x4 (&xr)[XV]) {
#pragma unroll
        for (int m = 0; m < XV; m++) {
            const int id = threadIdx.x + 256 * m;
            if (id < BN * 4) *reinterpret_cast<u32x4 *>(&xs[buf][0][0] + xs_off(id >> 2, id & 3)) = xr[m];
        }
    };

    constexpr int FB = MODE ? 4 : 1;                                     // 16-row blocks a wavefront multiplies
    f32x4 acc[FB][NB];
#pragma unroll
    for (int f = 0; f < FB; f++)
#pragma unroll
        for (int n = 0; n < NB; n++) acc[f][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // sources and activations requested three steps ahead (rings of four)
    constexpr int XD = 4, XL = XD - 1;
    Src<EXP> sw[4];
    u32x4 xr[XD][XV];
    src_load(kbeg, sw[0]);
    src_load(kbeg + 1, sw[1]);
    src_load(kbeg + 2, sw[2]);
#pragma unroll
    for (int k = 0; k < XL; k++) x_load(kbeg + k, xr[k]);
    __syncthreads();                                                     // the staged verbatim run

    auto step = [&](int k, auto S4) {
        constexpr int s4 = decltype(S4)::value;
        // rebuild this step's operand of the wavefront's 16 rows
        u32x4 w = lw_rebuild8<EXP>(sw[s4].s0, EXP ? sw[s4].s1 : 0u, sw[s4].lo, sw[s4].hi, a);
        const int32_t v = sw[s4].vr;
        if (v >= 0 && v < a.n_verbatim) {                                // rare: a stored segment
            const uint32_t cl = 32u * (k & 7) + 8u * q;
            w = staged && (uint32_t)v - v0 < v1 - v0
                    ? *reinterpret_cast<const u32x4 *>(&vs[(uint32_t)v - v0][cl & 63u])
                    : *reinterpret_cast<const u32x4 *>(a.verbatim + (int64_t)v * 64 + (cl & 63u));
        }
        if constexpr (MODE) as[k & 1][wave][lane] = w;
        x_store(k & 1, xr[s4 % XD]);
        if (k + 3 < kend) src_load(k + 3, sw[(s4 + 3) & 3]);
        if (k + XL < kend) x_load(k + XL, xr[(s4 + XL) % XD]);
        __syncthreads();
        const uint8_t *xb = &xs[k & 1][0][0];
        const int nb0 = MODE ? 16 * NB * wave : 0;                       // this wavefront's first batch column
        bf16x8 av[FB];
        if constexpr (MODE) {
#pragma unroll
            for (int f = 0; f < 4; f++) av[f] = __builtin_bit_cast(bf16x8, as[k & 1][f][lane]);
        } else {
            av[0] = __builtin_bit_cast(bf16x8, w);
        }
#pragma unroll
        for (int n = 0; n < NB; n++) {
            const u32x4 bv = *reinterpret_cast<const u32x4 *>(xb + xs_off(nb0 + 16 * n + j, q));
            const bf16x8 b = __builtin_bit_cast(bf16x8, bv);
#pragma unroll
            for (int f = 0; f < FB; f++) acc[f][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[f], b, acc[f][n], 0, 0, 0);
        }
    };
    for (int k = kbeg; k < kend; k += 4) {     // whole column blocks: 8 steps each
        step(k, std::integral_constant<int, 0>{});
        step(k + 1, std::integral_constant<int, 1>{});
        step(k + 2, std::integral_constant<int, 2>{});
        step(k + 3, std::integral_constant<int, 3>{});
    }

    // y^T rows r0 + 4q .. + 3 of batch column b0 + nb0 + 16n + j
    const int nb0 = MODE ? 16 * NB * wave : 0;
#pragma unroll
    for (int f = 0; f < FB; f++) {
        const int64_t r0 = row0 + 16 * (MODE ? f : wave) + 4 * q;
#pragma unroll
        for (int n = 0; n < NB; n++) {
            const int b = b0 + nb0 + 16 * n + j;
            if (b >= a.batch) continue;
            float *dst = a.splits > 1 ? a.part + ((int64_t)sz * a.batch + b) * a.rows : a.y + (int64_t)b * a.rows;
            *reinterpret_cast<f32x4 *>(dst + r0) = acc[f][n];
        }
    }
}

// y = the sum of the split partials, in split order (deterministic)
__global__ __launch_bounds__(256) void k_recon_reduce(const f32x4 *__restrict__ part, f32x4 *__restrict__ y,
                                                      int64_t n4, int splits)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    f32x4 v = part[i];
    for (int s = 1; s < splits; s++) v += part[(int64_t)s * n4 + i];
    y[i] = v;
}

template <bool EXP, int MODE, int NB>
hipError_t launch(const RArgs &a, hipStream_t s)
{
    constexpr int BN = MODE ? 64 * NB : 16 * NB;
    const int64_t gx = a.rows / 64;
    const int64_t gy = (a.batch + BN - 1) / BN;
    if (gx > 0x7FFFFFFF || gy > 65535 || a.splits < 1 || a.splits > 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_recon<EXP, MODE, NB>), dim3((unsigned)gx, (unsigned)gy, (unsigned)a.splits), dim3(256), 0,
                       s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    const int64_t n4 = (int64_t)a.batch * a.rows / 4;
    hipLaunchKernelGGL(k_recon_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const f32x4 *>(a.part), reinterpret_cast<f32x4 *>(a.y), n4, a.splits);
    return hipGetLastError();
}

template <bool EXP>
hipError_t launch_variant(const RArgs &a, int variant, hipStream_t s)
{
    switch (variant) {
    case 0: return launch<EXP, 0, 1>(a, s);
    case 1: return launch<EXP, 0, 2>(a, s);
    case 2: return launch<EXP, 0, 4>(a, s);
    case 3: return launch<EXP, 1, 2>(a, s);
    case 4: return launch<EXP, 1, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// variant: 0..2 = the rows split between the wavefronts, 16, 32 or 64 batch
// columns a workgroup; 3..4 = the batch split, 128 or 256 batch columns.
hipError_t lw_launch_recon(bool exponents, const uint32_t *src, const uint32_t *sm, const int32_t *vrank,
                           const uint32_t *vb_start, const uint16_t *verbatim, int64_t n_verbatim,
                           const uint8_t *palette, const uint16_t *x, float *y, int64_t rows, int64_t cols,
                           int batch, int variant, float *part, int splits, hipStream_t s)
{
    RArgs a;
    a.n_verbatim = n_verbatim;
    a.part = part;
    a.splits = splits;
    a.src = src;
    a.sm = sm;
    a.vrank = vrank;
    a.vb_start = vb_start;
    a.verbatim = verbatim;
    a.x = x;
    a.y = y;
    a.rows = rows;
    a.cols = cols;
    a.ncb = (int)(cols / 256);
    a.batch = batch;
    uint32_t t[4] = {0, 0, 0, 0};
    for (int i = 0; i < 16; i++) {
        const uint32_t e = palette ? palette[i] : 0u;
        const uint32_t tb = ((e >> 1) | (e << 7)) & 0xFFu;
        t[i >> 2] |= tb << (8 * (i & 3));
    }
    a.t03 = t[0];
    a.t47 = t[1];
    a.t8b = t[2];
    a.tcf = t[3];
    return exponents ? launch_variant<true>(a, variant, s) : launch_variant<false>(a, variant, s);
}
