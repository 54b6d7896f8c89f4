// rans.hip -- decode-only kernel of the rANS twin, the decode-cost ablation
// set beside the Huffman lane decoder ("LazyWeights", section "Decoder
// hardware", the comparison of Huffman and rANS decoders).
//
// Format (built by lw_rans_build): one frequency table per matrix scaled to
// 2^11 slots; one stream per tile row, or two (one per half of the row's
// columns), so a 64x256 tile is NS = 64 or 128 streams and a wavefront
// decodes a tile with one row per lane; a tile block is the NS head states
// followed by the 16-bit renormalisation chunks, chunk k of stream s at
// 16-bit unit NS k + s.  With two streams a row, a lane's two chains are
// independent and their steps interleave, hiding one chain's table latency
// behind the other's.
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One tile per wavefront: H streams per row (H = 1: the whole row; H = 2:
// one per half of its columns), lane l decoding row l's H streams, whose
// steps are independent and interleaved.
template <int SPR, int H, int RW>
__global__ __launch_bounds__(64 * RW) void k_rans_decode(const u32x4 *__restrict__ lut_g,
                                                         const uint32_t *__restrict__ tile_off,
                                                         const uint32_t *__restrict__ words, uint8_t *__restrict__ out,
                                                         uint32_t *__restrict__ final_state, int64_t nt, int ncb,
                                                         int64_t out_stride, int region)
{
    constexpr int NS = 64 * H, SPS = SPR / H;            // streams a tile, symbols a stream
    constexpr int SPARE = (NS / 2) * (CLAMP + 1);       // spare chunk rows, in words
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
        // a block is NS states plus whole rows of NS/2 words, and must leave the spare area
        if (n >= NS && n <= region - SPARE && ((n - NS) % (NS / 2)) == 0) nw = (int)n;
    }
    const u32x4 *src = reinterpret_cast<const u32x4 *>(words + off);
    for (int i = lane; i < nw / 4; i += 64) reinterpret_cast<u32x4 *>(blk)[i] = src[i];
    if (nw)
        for (int i = lane; i < SPARE; i += 64) blk[nw + i] = 0;
    __syncthreads();
    if (!nw) return;

    const uint32_t kt = (uint32_t)(nw - NS) / (NS / 2);
    const u32x2 *lut = reinterpret_cast<const u32x2 *>(lds);
    // byte address of stream s's chunk k: the block's chunk area + 2 (NS k + s)
    const char *cbase = reinterpret_cast<const char *>(blk + NS);
    uint32_t x[H], k[H];
#pragma unroll
    for (int h = 0; h < H; h++) {
        x[h] = blk[64 * h + lane];
        k[h] = 0;
    }
    const int64_t row = (t / ncb) * 64 + lane;
    uint8_t *drow = out + row * out_stride + (t % ncb) * SPR;
    for (int g = 0; g < SPS / GROUP; g++) {
        uint32_t e[H][GROUP];
#pragma unroll
        for (int j = 0; j < GROUP; j++) {
#pragma unroll
            for (int h = 0; h < H; h++) {
                if (j % CLAMP == 0) k[h] = min(k[h], kt);   // row kt is the first spare row
                const u32x2 ed = lut[x[h] & (LUT_SLOTS - 1)];
                uint32_t c = *reinterpret_cast<const uint16_t *>(cbase + 2u * (NS * k[h] + 64 * h + lane));
                asm volatile("" : "+v"(c));                 // keep the chunk read unconditional (no branch per symbol)
                uint32_t xx = (ed.x & 0xFFFFFFu) * (x[h] >> 11) + ed.y;
                const bool need = xx < RANS_L;
                x[h] = need ? (xx << 16) | c : xx;
                unsigned carry;
                k[h] = __builtin_addc(k[h], 0u, need ? 1u : 0u, &carry);
                e[h][j] = ed.x;
            }
        }
#pragma unroll
        for (int h = 0; h < H; h++) {
            uint32_t o[GROUP / 4];
#pragma unroll
            for (int q = 0; q < GROUP / 4; q++)
                o[q] = __builtin_amdgcn_perm(e[h][4 * q + 1], e[h][4 * q], 0x0C0C0703u) |
                       __builtin_amdgcn_perm(e[h][4 * q + 3], e[h][4 * q + 2], 0x07030C0Cu);
            reinterpret_cast<u32x4 *>(drow + h * SPS)[g] = u32x4{o[0], o[1], o[2], o[3]};
        }
    }
    if (final_state)
#pragma unroll
        for (int h = 0; h < H; h++) final_state[t * NS + 64 * h + lane] = x[h];
}

constexpr size_t lds_bytes(int rw, int region) { return sizeof(uint32_t) * ((size_t)LUT_WORDS + (size_t)rw * region); }

template <int SPR, int H, int RW>
hipError_t launch_rw(const uint32_t *lut, const uint32_t *tile_off, const uint32_t *words, uint8_t *out,
                     uint32_t *final_state, int64_t nt, int ncb, int64_t out_stride, int region, hipStream_t s)
{
    hipError_t e = lw_allow_lds<k_rans_decode<SPR, H, RW>>();
    if (e != hipSuccess) return e;
    const int64_t grid = (nt + RW - 1) / RW;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_rans_decode<SPR, H, RW>), dim3((unsigned)grid), dim3(64 * RW), lds_bytes(RW, region), s,
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

template <int SPR, int H>
hipError_t launch(const uint32_t *lut, const uint32_t *tile_off, const uint32_t *words, uint8_t *out,
                  uint32_t *final_state, int64_t nt, int ncb, int64_t out_stride, int max_tile_words, hipStream_t s)
{
    const int region = max_tile_words + 32 * H * (CLAMP + 1);
    const int lds = lw_device_lds_bytes();
    const int rw = lds > 0 ? pick_rw(region, (size_t)lds) : 0;
    if (rw == 4) return launch_rw<SPR, H, 4>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, region, s);
    if (rw == 6) return launch_rw<SPR, H, 6>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, region, s);
    if (rw == 8) return launch_rw<SPR, H, 8>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, region, s);
    return hipErrorNotSupported;
}

}  // namespace

hipError_t lw_launch_rans_decode(int spr, int halves, const uint32_t *lut, const uint32_t *tile_off,
                                 const uint32_t *words, uint8_t *out, uint32_t *final_state, int64_t nt, int ncb,
                                 int64_t out_stride, int max_tile_words, hipStream_t s)
{
    if (spr == 128 && halves == 1)
        return launch<128, 1>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, max_tile_words, s);
    if (spr == 256 && halves == 1)
        return launch<256, 1>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, max_tile_words, s);
    if (spr == 128 && halves == 2)
        return launch<128, 2>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, max_tile_words, s);
    if (spr == 256 && halves == 2)
        return launch<256, 2>(lut, tile_off, words, out, final_state, nt, ncb, out_stride, max_tile_words, s);
    return hipErrorInvalidValue;
}
