// rans.hip -- decode-only kernel of the rANS twin, the decode-cost ablation
// set beside the Huffman lane decoder ("LazyWeights", section "Decoder
// hardware", the comparison of Huffman and rANS decoders).
//
// Format (built by lw_rans_build): one frequency table per matrix scaled to
// 2^11 slots; one stream per tile row, so a 64x256 tile is 64 streams and a
// wavefront decodes a tile with one stream per lane; a tile block is the 64
// head states followed by the 16-bit renormalisation chunks, chunk k of row r
// at 16-bit unit 64k + r.
//
// Per symbol a lane does
//     (e, d) = lut[x mod 2^11]     e = f | symbol << 24, d = slot - cum
//     x      = f * (x >> 11) + d   (one v_mad_u32_u24: it reads only e's low 24 bits)
//     x      = x < 2^16 ? x << 16 | next chunk : x
// At most one chunk is needed per symbol (after the step x >= 32, so one
// 16-bit shift lifts it to at least 2^21 >= 2^16), so the chunk at the lane's
// read position is fetched every step, beside the table read, and kept only
// when the state fell below 2^16; the position advances by the compare's
// carry.  Unlike the Huffman decoder, where the symbol table read is off the
// lane's serial chain, here the table read is on it: the next slot depends
// on the looked-up frequency.  Symbols are packed four to a word with two
// byte permutes and an OR.
//
// A workgroup holds the 16 KB table and RW tile blocks in LDS; RW (4, 6 or
// 8 wavefronts) is chosen per launch to fit the most wavefronts in a CU's
// LDS, since with one stream per lane the chain's latency is hidden only by
// other wavefronts.  The read position is clamped once per 4 symbols to a
// zeroed spare area of 5 chunk rows after the block, so a corrupt stream
// decodes garbage but never reads outside its own LDS region.
#include <algorithm>

#include "lane_decode.hpp"

namespace {

constexpr uint32_t RANS_L = 1u << 16;
constexpr int LUT_SLOTS = 2048;
constexpr int LUT_WORDS = 2 * LUT_SLOTS; // (e, d) pairs
constexpr int GROUP = 16;                // symbols per output vector
constexpr int CLAMP = 4;                 // symbols per clamp of the read position
constexpr int SPARE_WORDS = 32 * (CLAMP + 1);

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int SPR, int RW>
__global__ __launch_bounds__(64 * RW) void k_rans_decode(const u32x4 *__restrict__ lut_g,
                                                         const uint32_t *__restrict__ tile_off,
                                                         const uint32_t *__restrict__ words, uint8_t *__restrict__ out,
                                                         uint32_t *__restrict__ final_state, int64_t nt, int ncb,
                                                         int64_t out_stride, int region)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    u32x4 *lut4 = reinterpret_cast<u32x4 *>(lds);
    for (int i = threadIdx.x; i < LUT_WORDS / 4; i += 64 * RW) lut4[i] = lut_g[i];

    const int64_t t = (int64_t)blockIdx.x * RW + wave;
    uint32_t *blk = lds + LUT_WORDS + wave * region;
    int64_t off = 0;
    int nw = 0;
    if (t < nt) {
        off = tile_off[t];
        const int64_t n = (int64_t)tile_off[t + 1] - off;
        // a block is 64 states plus whole rows of 32 words, and must leave the spare area
        if (n >= 64 && n <= region - SPARE_WORDS && ((n - 64) & 31) == 0) nw = (int)n;
    }
    const u32x4 *src = reinterpret_cast<const u32x4 *>(words + off);
    for (int i = lane; i < nw / 4; i += 64) reinterpret_cast<u32x4 *>(blk)[i] = src[i];
    if (nw)
        for (int i = lane; i < SPARE_WORDS; i += 64) blk[nw + i] = 0;
    __syncthreads();
    if (!nw) return;

    const uint32_t kt = (uint32_t)(nw - 64) >> 5;
    const u32x2 *lut = reinterpret_cast<const u32x2 *>(lds);
    // byte address of this lane's chunk k: the block's chunk area + 128 k + 2 lane
    const char *cbase = reinterpret_cast<const char *>(blk + 64) + 2 * lane;
    uint32_t k = 0;
    uint32_t x = blk[lane];
    const int64_t row = (t / ncb) * 64 + lane;
    u32x4 *dst = reinterpret_cast<u32x4 *>(out + row * out_stride + (t % ncb) * SPR);
    for (int g = 0; g < SPR / GROUP; g++) {
        uint32_t e[GROUP];
#pragma unroll
        for (int j = 0; j < GROUP; j++) {
            if (j % CLAMP == 0) k = min(k, kt);      // row kt is the first spare row
            const u32x2 ed = lut[x & (LUT_SLOTS - 1)];
            uint32_t c = *reinterpret_cast<const uint16_t *>(cbase + 128u * k);
            asm volatile("" : "+v"(c));              // keep the chunk read unconditional (no branch per symbol)
            x = (ed.x & 0xFFFFFFu) * (x >> 11) + ed.y;
            const bool need = x < RANS_L;
            x = need ? (x << 16) | c : x;
            unsigned carry;
            k = __builtin_addc(k, 0u, need ? 1u : 0u, &carry);
            e[j] = ed.x;
        }
        uint32_t o[GROUP / 4];
#pragma unroll
        for (int q = 0; q < GROUP / 4; q++)
            o[q] = __builtin_amdgcn_perm(e[4 * q + 1], e[4 * q], 0x0C0C0703u) |
                   __builtin_amdgcn_perm(e[4 * q + 3], e[4 * q + 2], 0x07030C0Cu);
        dst[g] = u32x4{o[0], o[1], o[2], o[3]};
    }
    if (final_state) final_state[t * 64 + lane] = x;
}

constexpr size_t lds_bytes(int rw, int region) { return sizeof(uint32_t) * ((size_t)LUT_WORDS + (size_t)rw * region); }

template <int SPR, int RW>
hipError_t launch_rw(const uint32_t *lut, const uint32_t *tile_off, const uint32_t *words, uint8_t *out,
                     uint32_t *final_state, int64_t nt, int ncb, int64_t out_stride, int region, hipStream_t s)
{
    hipError_t e = lw_allow_lds<k_rans_decode<SPR, RW>>();
    if (e != hipSuccess) return e;
    const int64_t grid = (nt + RW - 1) / RW;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_rans_decode<SPR, RW>), dim3((unsigned)grid), dim3(64 * RW), lds_bytes(RW, region), s,
                       reinterpret_cast<const u32x4 *>(lut), tile_off, words, out, final_state, nt, ncb, out_stride,
                       region);
    return hipGetLastError();
}

// Wavefronts per workgroup: the most resident wavefronts per CU (the table
// is shared by a workgroup's tiles), ties to the smaller workgroup.
inline int pick_rw(int region, size_t cu_lds)
{
    int best = 0, best_waves = 0;
    for (int rw : {4, 6, 8}) {
        const size_t b = lds_bytes(rw, region);
        if (b > cu_lds) continue;
        const int waves = rw * std::min<int>((int)(cu_lds / b), 32 / rw);
        if (waves > best_waves) { best = rw; best_waves = waves; }
    }
    return best;
}

template <int SPR>
hipError_t launch(const uint32_t *lut, const uint32_t *tile_off, const uint32_t *words, uint8_t *out,
                  uint32_t *final_state, int64_t nt, int ncb, int64_t out_stride, int max_tile_words, hipStream_t s)
{
    const int region = max_tile_words + SPARE_WORDS;
    const int lds = lw_device_lds_bytes();
    const int rw = lds > 0 ? pick_rw(region, (size_t)lds) : 0;
    if (rw == 4) return launch_rw<SPR, 4>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, region, s);
    if (rw == 6) return launch_rw<SPR, 6>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, region, s);
    if (rw == 8) return launch_rw<SPR, 8>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, region, s);
    return hipErrorNotSupported;
}

}  // namespace

hipError_t lw_launch_rans_decode(int spr, const uint32_t *lut, const uint32_t *tile_off, const uint32_t *words,
                                 uint8_t *out, uint32_t *final_state, int64_t nt, int ncb, int64_t out_stride,
                                 int max_tile_words, hipStream_t s)
{
    if (spr == 128)
        return launch<128>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, max_tile_words, s);
    if (spr == 256)
        return launch<256>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, max_tile_words, s);
    return hipErrorInvalidValue;
}
