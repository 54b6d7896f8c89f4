// bf16.hip -- fused exponent-decode + GEMV (batch 1..7) and decode-only for
// bf16 weights whose exponent byte is Huffman coded ("Unweight: Compressing
// LLM Weights for Faster Inference", sections "Understanding BF16 weight
// structure" and "The exponent's exploitable redundancy"), gfx950.
//
// A lane decodes palette indices with the same per-lane decoder as the
// quantised kernels (512 single symbols: tile rows 2l then 2l+1).  Payload
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
    c.rb = rb < a.n_rb ? rb : rb - 1;
    c.t = c.rb * a.n_cb + (c.wave_active ? c.cb : 0);
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

// Ordinal, in the verbatim store, of segment `bit` (4*row + segment) of tile t.
LW_DEV uint32_t lw_verbatim_ordinal(const KArgs &a, int64_t t, int bit)
{
    const uint32_t *vb = a.vb_bits + (size_t)t * 8;
    uint32_t n = a.vb_start[t];
    for (int w = 0; w < bit / 32; w++) n += __builtin_popcount(vb[w]);
    const uint32_t below = vb[bit / 32] & ((1u << (bit % 32)) - 1u);
    return n + __builtin_popcount(below);
}

template <int N8, int N16, int BATCH>
__global__ __launch_bounds__(256) void k_gemv_bf16(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const LdsLayout L = lds_layout(BATCH, a.max_words, false);
    const LaneCtx c = lane_ctx(a);
    const int S = a.max_words + 3;
    uint32_t *xs = reinterpret_cast<uint32_t *>(lds + L.x) + c.wave * BATCH * 128;
    const uint32_t xs_addr = (uint32_t)(size_t)xs;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + (c.wave * 2 + c.half) * S * 32;

    lw_stage_tab(lds, a.tab, a.min_len, a.max_len, false);
    if (c.wave_active) {
        const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
        lw_stage_tile(slots, a.words, w0, (w1 - w0) >> 5, c.l);
        const uint32_t *xg = reinterpret_cast<const uint32_t *>(a.x);
#pragma unroll
        for (int b = 0; b < BATCH; b++) {
            const uint32_t *xb = xg + (size_t)b * (a.cols / 2) + (size_t)c.cb * 128;
            xs[b * 128 + c.lane] = xb[c.lane];
            xs[b * 128 + c.lane + 64] = xb[c.lane + 64];
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
        if (ok) {
            struct XA {
                u32x2 v[BATCH];
                uint32_t sm;
            };
            auto run_row = [&](auto pc) {
                constexpr int p = decltype(pc)::value;
                const uint32_t *smrow = a.sm + (size_t)c.t * 4096 + (size_t)p * 64 * 32 + c.l;
                uint32_t ring[2][CHUNK];
                uint32_t pend = 0;
                auto run_chunk = [&](int ch, const uint32_t (&cur)[CHUNK]) {
                    auto fetch = [&](int g) {
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
                                acc[p][b] = lw_dot2_bf16(w2, j == 1 ? x.v[b].x : x.v[b].y, acc[p][b]);
                        } else {
                            pend = pay;
                        }
                    };
                    lw_decode_pipelined<N8, N16, CHUNK, XA, true>(
                        d, a, [](int j) { return (j & 1) ? (LW_TPAY_HI - LW_TPAY) : 0u; }, fetch, use);
                };
                lw_load_sm(ring[0], smrow, 0);
#pragma unroll
                for (int ch = 0; ch < 64 / CHUNK; ch += 2) {
                    lw_load_sm(ring[1], smrow, ch + 1);
                    run_chunk(ch, ring[0]);
                    if (ch + 2 < 64 / CHUNK) lw_load_sm(ring[0], smrow, ch + 2);
                    run_chunk(ch + 1, ring[1]);
                }
            };
            run_row(std::integral_constant<int, 0>{});
            run_row(std::integral_constant<int, 1>{});

            // verbatim segments of this lane's two rows (rare): replace the
            // placeholder weights' contribution by the stored values'
            const uint32_t bits = (a.vb_bits[(size_t)c.t * 8 + c.l / 4] >> (8 * (c.l % 4))) & 0xFFu;
            if (bits) {
                const uint16_t *xrow = a.x + (size_t)c.cb * 256;
                for (int q = 0; q < 8; q++) {
                    if (!((bits >> q) & 1u)) continue;
                    const int p = q >> 2, seg = q & 3;
                    const uint32_t ord = lw_verbatim_ordinal(a, c.t, 8 * c.l + q);
                    const uint16_t *v = a.verbatim + (size_t)ord * 64;
                    const uint32_t *smw = a.sm + (size_t)c.t * 4096 + (size_t)p * 64 * 32 + c.l;
                    for (int b = 0; b < BATCH; b++) {
                        float s = 0.f;
                        for (int k = 0; k < 64; k++) {
                            const int col = 64 * seg + k;
                            const uint32_t smb = (smw[(col / 4) * 32] >> (8 * (col % 4))) & 0xFFu;
                            const uint32_t ph = ((smb & 0x80u) << 8) | (a.pal0 << 7) | (smb & 0x7Fu);
                            const float wdiff = lw_bf16_to_f32(v[k]) - lw_bf16_to_f32(ph);
                            s += wdiff * lw_bf16_to_f32(xrow[(size_t)b * a.cols + col]);
                        }
                        if (p) acc[1][b] += s;
                        else acc[0][b] += s;
                    }
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < 2; p++)
#pragma unroll
                for (int b = 0; b < BATCH; b++) acc[p][b] = __builtin_nanf("");
        }
    }
    __syncthreads();                      // tiles no longer read: reuse for the reduction
    float *red = reinterpret_cast<float *>(lds + L.tiles);
#pragma unroll
    for (int p = 0; p < 2; p++)
#pragma unroll
        for (int b = 0; b < BATCH; b++)
            red[(c.wave * BATCH + b) * 128 + c.half * 64 + 2 * c.l + p] = c.lane_active ? acc[p][b] : 0.f;
    __syncthreads();
    uint32_t *last_flag = reinterpret_cast<uint32_t *>(lds + L.flag);
    lw_finish_rows<BATCH>(a, red, (int64_t)c.rbp * 128, c.g, c.rbp, WAVES, last_flag);
}

// Decode only: rebuild the bf16 matrix [rows][cols].
template <int N8, int N16>
__global__ __launch_bounds__(256) void k_decode_bf16(KArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const LdsLayout L = lds_layout(1, a.max_words, true);
    const LaneCtx c = lane_ctx(a);
    const int S = a.max_words + 3;
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + L.tiles) + (c.wave * 2 + c.half) * S * 32;
    lw_stage_tab(lds, a.tab, a.min_len, a.max_len, false);
    if (c.wave_active) {
        const uint32_t w0 = a.tile_off[c.t], w1 = a.tile_off[c.t + 1];
        lw_stage_tile(slots, a.words, w0, (w1 - w0) >> 5, c.l);
    }
    __syncthreads();
    if (!c.wave_active) return;
    LaneDec d;
    if (!lw_lane_init(d, lds, slots, c.l, a)) return;
    uint32_t *out = reinterpret_cast<uint32_t *>(a.out);
    struct XA {
        uint32_t sm;
    };
    auto run_row = [&](int p) {
        const uint32_t *smrow = a.sm + (size_t)c.t * 4096 + (size_t)p * 64 * 32 + c.l;
        uint32_t *orow = out + (((int64_t)c.rb * 64 + 2 * c.l + p) * a.cols + (int64_t)c.cb * 256) / 2;
        uint32_t ring[2][CHUNK];
        uint32_t pend = 0;
        auto run_chunk = [&](int ch, const uint32_t (&cur)[CHUNK]) {
            lw_decode_pipelined<N8, N16, CHUNK, XA, true>(
                d, a, [](int j) { return (j & 1) ? (LW_TPAY_HI - LW_TPAY) : 0u; },
                [&](int g) { return XA{cur[g]}; },
                [&](int g, int j, uint32_t pay, const XA &x) {
                    if (j & 1) {
                        const uint32_t w2 = (j == 1) ? lw_pair<0>(x.sm, pend, pay) : lw_pair<2>(x.sm, pend, pay);
                        if (c.lane_active) orow[2 * (ch * CHUNK + g) + (j >> 1)] = w2;
                    } else {
                        pend = pay;
                    }
                });
        };
        lw_load_sm(ring[0], smrow, 0);
#pragma unroll
        for (int ch = 0; ch < 64 / CHUNK; ch += 2) {
            lw_load_sm(ring[1], smrow, ch + 1);
            run_chunk(ch, ring[0]);
            if (ch + 2 < 64 / CHUNK) lw_load_sm(ring[0], smrow, ch + 2);
            run_chunk(ch + 1, ring[1]);
        }
    };
    run_row(0);
    run_row(1);
    if (a.lane_bits && c.lane_active) a.lane_bits[(size_t)c.t * 32 + c.l] = d.u - 31;
    // verbatim segments overwrite the placeholder weights (rare)
    const uint32_t bits = (a.vb_bits[(size_t)c.t * 8 + c.l / 4] >> (8 * (c.l % 4))) & 0xFFu;
    if (bits && c.lane_active) {
        uint16_t *o16 = reinterpret_cast<uint16_t *>(a.out);
        for (int q = 0; q < 8; q++) {
            if (!((bits >> q) & 1u)) continue;
            const int p = q >> 2, seg = q & 3;
            const uint32_t ord = lw_verbatim_ordinal(a, c.t, 8 * c.l + q);
            const int64_t row = (int64_t)c.rb * 64 + 2 * c.l + p;
            for (int k = 0; k < 64; k++)
                o16[row * a.cols + (int64_t)c.cb * 256 + 64 * seg + k] = a.verbatim[(size_t)ord * 64 + k];
        }
    }
}

template <int N8, int N16, int BATCH>
hipError_t launch_gemv(const KArgs &a, hipStream_t s)
{
    const LdsLayout L = lds_layout(BATCH, a.max_words, false);
    dim3 grid((unsigned)a.groups, (unsigned)((a.n_rb + 1) / 2));
    auto kern = k_gemv_bf16<N8, N16, BATCH>;
    hipError_t e = lw_allow_lds<k_gemv_bf16<N8, N16, BATCH>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(256), L.total, s, a);
    return hipGetLastError();
}

template <int N8, int N16>
hipError_t launch_decode(const KArgs &a, hipStream_t s)
{
    const LdsLayout L = lds_layout(1, a.max_words, true);
    dim3 grid((unsigned)a.groups, (unsigned)((a.n_rb + 1) / 2));
    auto kern = k_decode_bf16<N8, N16>;
    hipError_t e = lw_allow_lds<k_decode_bf16<N8, N16>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(256), L.total, s, a);
    return hipGetLastError();
}

template <int N8, int N16>
hipError_t gemv_batch(const KArgs &a, int batch, hipStream_t s)
{
    switch (batch) {
    case 1: return launch_gemv<N8, N16, 1>(a, s);
    case 2: return launch_gemv<N8, N16, 2>(a, s);
    case 3: return launch_gemv<N8, N16, 3>(a, s);
    case 4: return launch_gemv<N8, N16, 4>(a, s);
    case 5: return launch_gemv<N8, N16, 5>(a, s);
    case 6: return launch_gemv<N8, N16, 6>(a, s);
    case 7: return launch_gemv<N8, N16, 7>(a, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

hipError_t lw_launch_gemv_bf16(const KArgs &a, SadPlan p, int batch, hipStream_t s)
{
    switch (p.n8ops * 2 + p.n16ops) {
    case 0: return gemv_batch<0, 0>(a, batch, s);
    case 1: return gemv_batch<0, 1>(a, batch, s);
    case 2: return gemv_batch<1, 0>(a, batch, s);
    case 3: return gemv_batch<1, 1>(a, batch, s);
    case 4: return gemv_batch<2, 0>(a, batch, s);
    case 5: return gemv_batch<2, 1>(a, batch, s);
    }
    return hipErrorInvalidValue;
}

hipError_t lw_launch_decode_bf16(const KArgs &a, SadPlan p, hipStream_t s)
{
    switch (p.n8ops * 2 + p.n16ops) {
    case 0: return launch_decode<0, 0>(a, s);
    case 1: return launch_decode<0, 1>(a, s);
    case 2: return launch_decode<1, 0>(a, s);
    case 3: return launch_decode<1, 1>(a, s);
    case 4: return launch_decode<2, 0>(a, s);
    case 5: return launch_decode<2, 1>(a, s);
    }
    return hipErrorInvalidValue;
}
