// lane_decode.hpp -- the per-lane Huffman decoder shared by the gfx950 kernels.
//
// "LazyWeights", section "3 . Decode on demand" and Fig. 3(b): each lane
// compares an 11-bit peek against per-length limits (no 2048-entry table),
// adds the code length's offset to index the symbol table, and shifts its
// buffer by the length.  Here one lane of a wavefront is one lane stream.
//
// Layout: a tile's interleaved words are staged in LDS as `slots` rows of 32
// dwords, slot j+1 holding word row j (slot 0 is a pad row before the stream,
// the last slot a pad row after it).  A lane keeps u = bitpos + 31, so the two
// words that hold bits [bitpos, bitpos+32) are slots u>>5 and (u>>5)+1, and
// the left-justified 32-bit window is their concatenation shifted left by
// bitpos mod 32 (v_alignbit with shift ~u mod 32).  Comparing the window with
// limit << 21 is the 11-bit peek comparison; the count r of limits passed
// gives the length min_len + r.  Bits past a lane's last code are don't-care
// (prefix property), and the slots bound every read of a valid stream.
#ifndef LW_LANE_DECODE_HPP
#define LW_LANE_DECODE_HPP

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LW_DEV __device__ __forceinline__

// Tables staged in LDS at the start of every decoding workgroup.
struct LdsTab {
    uint32_t pay[256];       // payload per canonical index
    uint32_t pay_hi[256];    // second payload (Q6 odd column / bf16 high half / symbol value)
    uint32_t len[16];        // code length per comparison count
    int32_t base[16];        // offset[len] - first[len] per comparison count
};

template <int NCMP>
LW_DEV uint32_t lw_count_limits(uint32_t win, const uint32_t *lim)
{
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < NCMP; i++) r += (win >= lim[i]) ? 1u : 0u;
    return r;
}

// Decode one symbol of the lane whose slot-0 word is lane_words[0] (stride
// 32 dwords between slots).  Returns the canonical index; advances u.
template <int NCMP>
LW_DEV uint32_t lw_decode_step(const uint32_t *lane_words, uint32_t &u, const uint32_t *lim,
                               const LdsTab &tab)
{
    const uint32_t slot = u >> 5;
    const uint32_t a = lane_words[slot * 32];
    const uint32_t b = lane_words[slot * 32 + 32];
    const uint32_t win = __builtin_amdgcn_alignbit(a, b, ~u);
    const uint32_t r = lw_count_limits<NCMP>(win, lim);
    const uint32_t len = tab.len[r];
    const int32_t base = tab.base[r];
    u += len;
    return (uint32_t)((int32_t)(win >> (32u - len)) + base);
}

LW_DEV uint32_t lw_wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

LW_DEV float lw_half_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFF)); }
LW_DEV float lw_half_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

typedef _Float16 lw_half2 __attribute__((ext_vector_type(2)));

LW_DEV float lw_dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(lw_half2, a), __builtin_bit_cast(lw_half2, b), c, false);
}

// sum over the 64 lanes of a wavefront
LW_DEV float lw_wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Stage the tables of a bundle into LDS (all threads of the block).
LW_DEV void lw_stage_tab(LdsTab &t, const lw_gputab *g, bool symval_as_hi)
{
    for (int i = threadIdx.x; i < 256; i += blockDim.x) {
        t.pay[i] = g->payload[i];
        t.pay_hi[i] = symval_as_hi ? g->symval[i] : g->payload_hi[i];
    }
    for (int i = threadIdx.x; i < 16; i += blockDim.x) {
        t.len[i] = g->len[i];
        t.base[i] = g->base[i];
    }
}

// Copy one tile block (W word rows) into LDS slots 1..W, by the 32 lanes l of
// a half-wave; 16 bytes per lane per step.
LW_DEV void lw_stage_tile(uint32_t *slots, const uint32_t *words, uint32_t w0, uint32_t nrows, int l)
{
    const uint4 *src = reinterpret_cast<const uint4 *>(words + w0);
    uint4 *dst = reinterpret_cast<uint4 *>(slots + 32);
    const uint32_t n = nrows * 8u;
    for (uint32_t i = (uint32_t)l; i < n; i += 32u) dst[i] = src[i];
}

#endif
