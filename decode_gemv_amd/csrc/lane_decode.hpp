// lane_decode.hpp -- the per-lane Huffman decoder shared by the gfx950 kernels.
//
// "LazyWeights", section "3 . Decode on demand" and Fig. 3(b): a lane finds
// a code's length from the next 11 bits of its stream by comparison with one
// bound per length (rather than a 2048-entry lookup), reads the symbol at that
// length's base position plus the code's rank, and advances by the length.  Here one lane of a wavefront is one lane stream.
//
// Words.  A tile's interleaved words are staged in LDS as rows of 32 dwords
// ("slots"): slot j+1 holds word row j, slot 0 and the last two slots are
// pads.  With u = bitpos + 31, the three words starting at slot u>>5 hold
// bits [bitpos, bitpos + 64) and two v_alignbit by ~u give a 64-bit
// left-justified register window (hi, lo).  A lane keeps un = ~u itself, so
// the shift is the register and the slot address is one shift-or and one
// subtraction: 128 (u >> 5) = -4 - ((un << 2) | 124).  One window serves four symbols:
// after three codes of at most 11 bits, 31 bits of it are still valid, more
// than the 11-bit peek needs.  So the LDS read sits on the lane's serial
// chain once per four symbols.
//
// Length.  For sorted limits c_i and an integer peek p,
//     |p - (c_i - 1)| - |p - c_i| = 2 [p >= c_i] - 1,
// so two sums of absolute differences count the limits the peek has passed:
// v_sad_u8 handles four limits per instruction on bytes, v_sad_u16 two on
// 16-bit halves.  A limit of a length <= 8 is a multiple of 8, so it compares
// exactly on the top 8 peek bits (floor(p / 8)).  A limit c of length 9 or 10
// is a multiple of 4 or 2: with k = (8 - c) mod 8, p >= c exactly when
// floor((p + k) / 8) >= (c + k) / 8, the top byte of the peek plus k << 21
// (a saturating add: k never carries a valid comparison past 2047).  So one
// v_perm_b32 gathers, per byte, the top byte of the peek or of the peek plus
// k, and two v_sad_u8 pairs compare up to eight limits (the residue plans;
// a table with two residues besides 0 gives each pair its own register).
// Tables with more than eight comparisons take the general plan: byte pairs
// on the top byte and one v_sad_u16 pair on the top 16 window bits.  With the
// accumulator chosen as K = PBASE - 2*min_len - n, the difference of the two
// sums is
//     A = PBASE - 2*len,
// which is at once the LDS address of the 16-bit entry of that length (the
// symbol-table base offset[len] - first[len], pre-scaled) and, shifted right
// by one, a shift amount s = PBASE/2 - len whose low five bits are 32 - len:
//     code = hi >> s,  window <<= len  ==  alignbit(hi, lo, s), alignbit(lo, 0, s).
// Bits past a lane's last code are don't-care (prefix property); the slots
// bound every read of a valid stream.
//
// Compact tables (at most four code lengths, the three shorter <= 8: what
// the builder makes).  One v_sad_u8 pair compares the top 8 peek bits with
// the three limits, and the accumulator makes A = CSEL - 2r for r limits
// passed.  A + 1 is the LDS address of the base entry of the r-th used
// length, and A is at once a v_perm_b32 selector into an 8-byte table held
// in two SGPRs: its low byte 7 - 2r picks the byte -length(r) mod 256, its
// second byte (at least 13) makes 0xFF, and its two zero upper bytes pick
// table byte 0, which holds 0xFF.  So the shift is s = -len exactly: its low
// five bits are 32 - len, and the lengths of a group sum without a mask.
//
// Sparse plan (a table with absent lengths, whose used lengths fit two SAD
// pairs with one residue where the whole length range does not: the bf16
// exponent tables).  The pairs compare the limits of the used lengths only
// (a residue r on the peek minus r << 21, saturating at 0: p >= c exactly
// when floor((p - r)/8) >= (c - r)/8, which holds for limits up to 2047),
// and A = SBASE - 2r for r limits passed: the LDS address of that count's
// base entry.  The low byte of A >> 1 is 7 - r, a v_perm_b32 selector into
// an 8-byte table of -len mod 256 per count; the shift's upper bytes are
// other table bytes, which shifts ignore, and the low byte of a group's sum
// of shifts, sign-extended, is -sum(len) (at most 44).
#ifndef LW_LANE_DECODE_HPP
#define LW_LANE_DECODE_HPP

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"

#define LW_DEV __device__ __forceinline__

// Host: the current device's largest LDS allocation per workgroup (cached
// per device; 0 if the query fails).
inline int lw_device_lds_bytes()
{
    constexpr int MAXDEV = 64;
    static std::once_flag once[MAXDEV];
    static int bytes[MAXDEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAXDEV) return 0;
    std::call_once(once[dev], [dev]() {
        if (hipDeviceGetAttribute(&bytes[dev], hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            bytes[dev] = 0;
    });
    return bytes[dev];
}

// Host: the current device's compute-unit count (cached per device; 0 if the
// query fails).
inline int lw_device_cu_count()
{
    constexpr int MAXDEV = 64;
    static std::once_flag once[MAXDEV];
    static int cus[MAXDEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAXDEV) return 0;
    std::call_once(once[dev], [dev]() {
        if (hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus[dev] = 0;
    });
    return cus[dev];
}

// Host: whether a grid of one wavefront per tile is resident at once (at
// most four wavefronts a SIMD): 1 or 0, the kernels' `ramp` argument.
inline int lw_resident_ramp(int64_t waves)
{
    const int cus = lw_device_cu_count();
    return cus > 0 && waves <= 16 * (int64_t)cus ? 1 : 0;
}

// Host: allow kernel KERN the device's largest dynamic LDS allocation, once
// per device.  The limit is a permission, not an allocation (a launch still
// reserves only what it asks for), so raising it to the maximum once keeps
// the runtime call off the launch path and can never be lowered by a
// concurrent caller.
template <auto KERN>
inline hipError_t lw_allow_lds()
{
    constexpr int MAXDEV = 64;
    static std::once_flag once[MAXDEV];
    static hipError_t result[MAXDEV];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev]() {
        int bytes = 0;
        result[dev] = hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (result[dev] == hipSuccess)
            result[dev] = hipFuncSetAttribute((const void *)KERN, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    });
    return result[dev];
}

// LDS layout common to all decoding kernels (byte offsets)
#define LW_PBASE LW_PLAN_PBASE   // length entries at PBASE - 2*len, len = 1..11
#define LW_TPAY 1024u        // payload per canonical index, u32[256]
#define LW_TPAY_HI 2048u     // second payload, u32[256]
#define LW_CSEL LW_PLAN_CSEL     // compact tables: selector of count r CSEL - 2r, its base entry at CSEL + 1 - 2r
#define LW_SBASE LW_PLAN_SBASE   // sparse plan: base entry of count r at SBASE - 2r
#define LW_TAB_BYTES 3584u

LW_DEV uint32_t lw_wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

LW_DEV float lw_half_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFF)); }
LW_DEV float lw_half_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

typedef _Float16 lw_half2 __attribute__((ext_vector_type(2)));

LW_DEV float lw_dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(lw_half2, a), __builtin_bit_cast(lw_half2, b), c, false);
}

// v + v of the lane that DPP control CTRL names (all rows and banks)
template <int CTRL>
LW_DEV float lw_dpp_add(float v)
{
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of W lanes (W a power of two, at most 64, every
// lane of a group active), the group's sum in each of its lanes: DPP steps
// inside rows of 16 lanes (pairs, quads, eights by the half-row mirror,
// sixteens by rotating the row by 8), LDS permutes across rows.
template <int W>
LW_DEV float lw_group_sum(float v);

// Sum over the 64 lanes of a wavefront (every lane active), the same value
// in every lane: four DPP steps sum each row of 16 lanes (pairs, quads,
// eights by the half-row mirror, rows by the row mirror), then the four row
// sums are read from lanes 0, 16, 32 and 48.  No LDS round trip.
LW_DEV float lw_wave_sum(float v)
{
    v = lw_dpp_add<0xB1>(v);              // quad_perm [1,0,3,2]
    v = lw_dpp_add<0x4E>(v);              // quad_perm [2,3,0,1]
    v = lw_dpp_add<0x141>(v);             // row_half_mirror
    v = lw_dpp_add<0x140>(v);             // row_mirror
    const int i = __builtin_bit_cast(int, v);
    auto lane = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(i, l)); };
    return (lane(0) + lane(16)) + (lane(32) + lane(48));
}

template <int W>
LW_DEV float lw_group_sum(float v)
{
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group of 1 to 64 lanes, a power of two");
    if constexpr (W >= 2) v = lw_dpp_add<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v = lw_dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v = lw_dpp_add<0x141>(v);   // row_half_mirror
    if constexpr (W >= 16) v = lw_dpp_add<0x128>(v);  // row_ror:8
    if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// LDS accessed by byte address (the kernels allocate only dynamic LDS, so
// the dynamic area starts at the workgroup's LDS address lb, normally 0;
// lb is folded into the table entries and the SAD offset so that the hot
// loop adds no base).
typedef __attribute__((address_space(3))) const int16_t lw_lds_i16;
typedef __attribute__((address_space(3))) const uint32_t lw_lds_u32;

LW_DEV uint32_t lw_ld32(uint32_t addr) { return *(lw_lds_u32 *)(size_t)addr; }
LW_DEV int32_t lw_ld16s(uint32_t addr) { return *(lw_lds_i16 *)(size_t)addr; }

// Split-phase staging.  A kernel's prologue first issues every global load
// it needs (tile offsets first, since the tile words depend on them; then the
// decoder table, scales and activations; then the tile words) and only then
// writes LDS, through address-space-3 pointers so that no store can be taken
// to alias a later load.  The prologue then costs the tile-offset and tile-word
// round trips instead of one round trip per kind of data.
typedef __attribute__((address_space(3))) uint32_t lw_lds_w32;
typedef __attribute__((address_space(3))) int16_t lw_lds_w16;
typedef uint32_t lw_u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) lw_u32x4 lw_lds_w128;

struct LwTabRegs {
    uint32_t pay, pay2;
    int32_t ent;
};

// whether a plan indexes the compact tables (length from a byte table)
template <int PLAN>
constexpr bool lw_compact() { return PLAN == LW_P_COMPACT; }
// whether a plan counts the used lengths only (length from a byte table)
template <int PLAN>
constexpr bool lw_sparse() { return PLAN == LW_P_S2K; }

// thread tid (< 256) fetches payload entry tid of both tables and length
// entry min(tid, max_len - min_len) (compact tables: the base of count
// min(tid, ncmp), from the kernel arguments; the sparse plan: the base of
// the length that count min(tid, ncmp) stands for, byte 7 - count of the
// byte table).  Loads and stores are unconditional: a load the compiler
// sinks into a divergent branch is waited on together with every load
// issued before it.
template <int PLAN>
LW_DEV LwTabRegs lw_tab_fetch(const KArgs &a, bool symval_second)
{
    LwTabRegs r;
    const int tid = threadIdx.x;
    const lw_gputab *g = a.tab;
    r.pay = g->payload[tid & 255];
    r.pay2 = symval_second ? g->symval[tid & 255] : g->payload_hi[tid & 255];
    if constexpr (lw_compact<PLAN>()) {
        const int i = min(tid, a.ncmp);
        r.ent = i == 0 ? a.cbase[0] : i == 1 ? a.cbase[1] : i == 2 ? a.cbase[2] : a.cbase[3];
    } else if constexpr (lw_sparse<PLAN>()) {
        const int i = min(tid, a.ncmp);   // ncmp <= 7
        const uint32_t nb = i < 4 ? a.lut_hi >> (8 * (3 - i)) : a.lut_lo >> (8 * (7 - i));   // -len mod 256
        r.ent = g->base[((256u - (nb & 0xFFu)) & 0xFFu) - (uint32_t)a.min_len];
    } else {
        r.ent = g->base[min(tid, a.max_len - a.min_len)];   // threads past the last entry repeat it
    }
    return r;
}

template <int PLAN>
LW_DEV void lw_tab_put(uint8_t *lds, const LwTabRegs &r, const KArgs &a)
{
    const uint32_t lb = (uint32_t)(size_t)lds;
    const int tid = threadIdx.x;          // workgroups have 256 threads: one entry each, unconditionally
    *(lw_lds_w32 *)(size_t)(lb + LW_TPAY + 4u * (tid & 255)) = r.pay;
    *(lw_lds_w32 *)(size_t)(lb + LW_TPAY_HI + 4u * (tid & 255)) = r.pay2;
    const int16_t v = (int16_t)((int32_t)lb + (int32_t)LW_TPAY + 4 * r.ent);   // repeated stores write the same value
    if constexpr (lw_compact<PLAN>())
        *(lw_lds_w16 *)(size_t)(lb + LW_CSEL + 1u - 2u * (uint32_t)min(tid, a.ncmp)) = v;
    else if constexpr (lw_sparse<PLAN>())
        *(lw_lds_w16 *)(size_t)(lb + LW_SBASE - 2u * (uint32_t)min(tid, a.ncmp)) = v;
    else
        *(lw_lds_w16 *)(size_t)(lb + LW_PBASE - 2u * (uint32_t)(a.min_len + min(tid, a.max_len - a.min_len))) = v;
}

// A wavefront stages one tile: lw_tile_fetch64 loads the first 64 word rows
// of the tile block (8 x 16 bytes per lane), lw_tile_put64 stores them into
// slots 1.. and stages any further rows in batches of 64.  Indices past the
// block are clamped to its last vector, so no load or store is predicated.
struct LwTileRegs64 {
    lw_u32x4 v[8];
};

LW_DEV void lw_tile_fetch64(const uint32_t *words, uint32_t w0, uint32_t nrows, int lane, LwTileRegs64 &r)
{
    const lw_u32x4 *src = reinterpret_cast<const lw_u32x4 *>(words + w0);
    const uint32_t n = nrows * 8u;
#pragma unroll
    for (int i = 0; i < 8; i++) r.v[i] = src[min((uint32_t)lane + 64u * i, n - 1u)];
}

LW_DEV void lw_tile_put64(uint32_t *slots, const uint32_t *words, uint32_t w0, uint32_t nrows, int lane,
                          const LwTileRegs64 &r)
{
    const uint32_t base = (uint32_t)(size_t)(slots + 32);      // slot 1
    const uint32_t n = nrows * 8u;
#pragma unroll
    for (int i = 0; i < 8; i++)
        *(lw_lds_w128 *)(size_t)(base + 16u * min((uint32_t)lane + 64u * i, n - 1u)) = r.v[i];
    const lw_u32x4 *src = reinterpret_cast<const lw_u32x4 *>(words + w0);
    for (uint32_t b0 = 512u; b0 < n; b0 += 512u) {            // long lanes: more batches
        lw_u32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = src[min(b0 + (uint32_t)lane + 64u * i, n - 1u)];
#pragma unroll
        for (int i = 0; i < 8; i++)
            *(lw_lds_w128 *)(size_t)(base + 16u * min(b0 + (uint32_t)lane + 64u * i, n - 1u)) = v[i];
    }
}

// Visit every verbatim segment of bf16 tile t ("Unweight": a 64-weight row
// segment holding an exponent outside the palette is stored whole), the 64
// lanes of the wavefront together: for tile row `row` and segment `seg`,
// lane k gets column col = 64*seg + k, the stored bf16 weight vv and the
// placeholder weight ph the stream decoded there (palette index 0 joined
// with the column's sign and mantissa).  Segments are visited in bitmap
// order (bit 4*row + seg), which is their order in the verbatim store, so
// the store index is a running count from vb_start[t].  The loop is
// wave-uniform; at N(0, 0.02) weights a tile holds about one such segment.
template <class F>
LW_DEV void lw_verbatim_visit(const KArgs &a, int64_t t, int lane, F f)
{
    const uint32_t words = a.vb_bits[(size_t)t * 8 + (lane & 7)];    // lanes 0..7: the tile's 256-bit map
    uint32_t ord = a.vb_start[t];
    for (int w = 0; w < 8; w++) {
        uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)words, w);
        while (bits) {
            const int bit = 32 * w + __builtin_ctz(bits);
            bits &= bits - 1u;
            const int row = bit >> 2, seg = bit & 3, col = 64 * seg + lane;
            const uint32_t vv = a.verbatim[(size_t)ord * 64 + lane];
            ord++;
            const uint32_t smw = a.sm[(size_t)t * 4096 + (size_t)(row & 1) * 64 * 32 + (size_t)(col / 4) * 32 + (row >> 1)];
            const uint32_t smb = (smw >> (8 * (col % 4))) & 0xFFu;
            const uint32_t ph = ((smb & 0x80u) << 8) | (a.pal0 << 7) | (smb & 0x7Fu);
            f(row, col, vv, ph);
        }
    }
}

// One lane's decoder state.
struct LaneDec {
    uint32_t wref;               // LDS byte address of this lane's word in slot 0, minus 4
    uint32_t un;                 // ~(bit position + 31)
    uint32_t k;                  // SAD offset including the LDS base
    uint32_t lut_lo;             // low word of the compact tables' shift bytes
    uint32_t xk[2];              // residue plans: the constants added to the peek
    uint32_t ubias;              // 4 * (lb/2 + PBASE/2): what four shifts s add beyond the code lengths
    LW_DEV void advance(uint32_t bits) { un -= bits; }
    LW_DEV uint32_t bitpos() const { return ~un - 31u; }
};

// peek + k with unsigned saturation (one v_add_u32 with the clamp bit)
LW_DEV uint32_t lw_add_sat(uint32_t v, uint32_t k)
{
    uint32_t r;
    asm("v_add_u32_e64 %0, %1, %2 clamp" : "=v"(r) : "v"(v), "v"(k));
    return r;
}

// peek - k, saturating at 0 (one v_sub_u32 with the clamp bit)
LW_DEV uint32_t lw_sub_sat(uint32_t v, uint32_t k)
{
    uint32_t r;
    asm("v_sub_u32_e64 %0, %1, %2 clamp" : "=v"(r) : "v"(v), "v"(k));
    return r;
}

// Count the limits the window's peek has passed; returns A = lb + PBASE - 2*len
// (compact tables: A = lb + CSEL - 2r, the sparse plan: A = lb + SBASE - 2r,
// for r limits passed).  xk holds the
// residue plans' additive constants in vector registers (see LaneDec).
template <int PLAN>
LW_DEV uint32_t lw_count(uint32_t hi, uint32_t k, const uint32_t (&xk)[2], const KArgs &a)
{
    uint32_t s1 = 0, s2 = k;
    if constexpr (PLAN == LW_P_COMPACT) {
        const uint32_t p8 = __builtin_amdgcn_perm(hi, hi, 0x03030303u);
        s1 = __builtin_amdgcn_sad_u8(p8, a.c8m1[0], s1);
        s2 = __builtin_amdgcn_sad_u8(p8, a.c8[0], s2);
    } else if constexpr (PLAN == LW_P_GEN) {
        const uint32_t p8 = __builtin_amdgcn_perm(hi, hi, 0x03030303u);
        const uint32_t p16 = __builtin_amdgcn_perm(hi, hi, 0x03020302u);
        s1 = __builtin_amdgcn_sad_u16(p16, a.c16m1, s1);
        s2 = __builtin_amdgcn_sad_u16(p16, a.c16, s2);
        s1 = __builtin_amdgcn_sad_u8(p8, a.c8m1[1], s1);
        s2 = __builtin_amdgcn_sad_u8(p8, a.c8[1], s2);
        s1 = __builtin_amdgcn_sad_u8(p8, a.c8m1[0], s1);
        s2 = __builtin_amdgcn_sad_u8(p8, a.c8[0], s2);
    } else {
        uint32_t x1, x2;
        if constexpr (PLAN == LW_P_R2) {
            x1 = __builtin_amdgcn_perm(hi, hi, 0x03030303u);
        } else if constexpr (PLAN == LW_P_S2K) {
            x1 = __builtin_amdgcn_perm(lw_sub_sat(hi, xk[0]), hi, a.xsel[0]);   // the residue subtracted
        } else {
            x1 = __builtin_amdgcn_perm(lw_add_sat(hi, xk[0]), hi, a.xsel[0]);
        }
        if constexpr (PLAN == LW_P_R2X2)
            x2 = __builtin_amdgcn_perm(lw_add_sat(hi, xk[1]), hi, a.xsel[1]);
        else
            x2 = x1;
        s1 = __builtin_amdgcn_sad_u8(x1, a.c8m1[0], s1);
        s2 = __builtin_amdgcn_sad_u8(x1, a.c8[0], s2);
        s1 = __builtin_amdgcn_sad_u8(x2, a.c8m1[1], s1);
        s2 = __builtin_amdgcn_sad_u8(x2, a.c8[1], s2);
    }
    return s2 - s1;
}

// Software-pipelined decode of NG (even) groups of four symbols of one lane
// stream.  LDS reads complete in issue order, so the loop keeps only the next
// window read on the serial chain: in step g it decodes group g (VALU only),
// issues the window read of group g+1, the payload reads (and fetch(g-1),
// the caller's other LDS operands) of group g-1 and the length-entry reads
// of group g, and hands group g-2 to use(group, j, payload, aux).  Pipeline
// registers are double-buffered by group parity and the loop is unrolled by
// two, so every buffer index is a compile-time constant (no register moves).
// pay_off(j) selects the payload table.  Scheduling barriers keep the issue
// order; the extra window read after the last group stays inside the staged
// slots.
template <int PLAN, int NG, class Aux, bool UNROLL_ALL = false, class PayOff, class Fetch, class Use>
LW_DEV void lw_decode_pipelined(LaneDec &d, const KArgs &a, PayOff pay_off, Fetch fetch, Use use)
{
    static_assert(NG % 2 == 0 && NG >= 4, "groups must be even");
    constexpr bool CMP = lw_compact<PLAN>(), SPR = lw_sparse<PLAN>();
    uint32_t wa, wb, wc;
    uint32_t code[2][4], A[2][4], base[2][4], pay[2][4];
    Aux aux[2];
    auto issue_window = [&]() {
        const uint32_t p = d.wref - ((d.un << 2) | 124u);    // slot u >> 5, 128 bytes per slot
        wa = lw_ld32(p);
        wb = lw_ld32(p + 128);
        wc = lw_ld32(p + 256);
    };
    // One group: align a 64-bit window (hi, lo) at the group's first bit,
    // then peek each symbol at its offset o within it.  s_j is -len_j
    // (compact tables) or bias - len_j with bias = lb/2 + 512 a multiple of
    // 64, so the running sum t of the s before symbol j is -o modulo 64.
    // Symbols 1 and 2 sit at most 22 bits in: one alignbit by t (which reads
    // t mod 32 = 32 - o) takes their peek, all 32 bits of it from the window.
    // Symbol 3 can sit 33 bits in, past one alignment; its peek is symbol
    // 2's advanced by symbol 2's length (an alignbit of (peek, 0) by s, whose
    // low five bits are 32 - len), which leaves 32 - len >= 21 bits from the
    // window: every plan reads at most the top 16 bits of a peek.
    auto decode_group = [&](int q) {
        const uint32_t sh = d.un;
        const uint32_t hi = __builtin_amdgcn_alignbit(wa, wb, sh), lo = __builtin_amdgcn_alignbit(wb, wc, sh);
        uint32_t t = 0, prev = 0, sprev = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            uint32_t peek;
            if (j == 0) peek = hi;
            else if (j < 3) peek = __builtin_amdgcn_alignbit(hi, lo, t);
            else peek = __builtin_amdgcn_alignbit(prev, 0u, sprev);
            const uint32_t Aj = lw_count<PLAN>(peek, d.k, d.xk, a);
            const uint32_t s = CMP   ? __builtin_amdgcn_perm(a.lut_hi, d.lut_lo, Aj)
                               : SPR ? __builtin_amdgcn_perm(a.lut_hi, d.lut_lo, Aj >> 1)
                                     : Aj >> 1;
            A[q][j] = Aj;
            code[q][j] = peek >> (s & 31u);
            t += s;
            prev = peek;
            sprev = s;
        }
        if constexpr (CMP)
            d.un += t;                    // t = -sum(len) exactly
        else if constexpr (SPR)
            d.un += (uint32_t)((int32_t)(t << 24) >> 24);   // the low byte of t is -sum(len) mod 256, sum <= 44
        else
            d.un += t - d.ubias;          // t - ubias = -sum(len)
    };
    auto issue_payloads = [&](int q, int g) {
#pragma unroll
        for (int j = 0; j < 4; j++)
            pay[q][j] = lw_ld32((uint32_t)((int32_t)(code[q][j] << 2) + (int32_t)base[q][j]) + pay_off(j));
        aux[q] = fetch(g);
    };
    auto issue_params = [&](int q) {
#pragma unroll
        for (int j = 0; j < 4; j++) base[q][j] = (uint32_t)lw_ld16s(A[q][j] + (CMP ? 1u : 0u));
    };
    auto use_group = [&](int q, int g) {
#pragma unroll
        for (int j = 0; j < 4; j++) use(g, j, pay[q][j], aux[q]);
    };
#define LW_FENCE() __builtin_amdgcn_sched_barrier(0)
    issue_window();
    LW_FENCE();
    decode_group(0);           // group 0
    LW_FENCE();
    issue_window();
    LW_FENCE();
    issue_params(0);
    LW_FENCE();
    decode_group(1);           // group 1
    LW_FENCE();
    issue_window();
    LW_FENCE();
    issue_payloads(0, 0);
    LW_FENCE();
    issue_params(1);
    LW_FENCE();
    constexpr int UNROLL = UNROLL_ALL ? NG : 1;
#pragma unroll UNROLL
    for (int g = 2; g < NG; g += 2) {
        decode_group(0);       // group g (even)
        LW_FENCE();
        issue_window();        // group g+1
        LW_FENCE();
        issue_payloads(1, g - 1);
        LW_FENCE();
        use_group(0, g - 2);
        LW_FENCE();
        issue_params(0);
        LW_FENCE();
        decode_group(1);       // group g+1 (odd)
        LW_FENCE();
        issue_window();        // group g+2 (past the end at the last step: in bounds)
        LW_FENCE();
        issue_payloads(0, g);
        LW_FENCE();
        use_group(1, g - 1);
        LW_FENCE();
        issue_params(1);
        LW_FENCE();
    }
    issue_payloads(1, NG - 1);
    use_group(0, NG - 2);
    use_group(1, NG - 1);
#undef LW_FENCE
}

// s_setprio P when `on` (wave-uniform) is nonzero.  The test and the skip
// sit inside one asm statement, so an unrolled decode loop around it stays
// one basic block (a branch there splits its scheduling and register
// allocation).
template <int P>
LW_DEV void lw_progress_priority(int on)
{
    asm volatile("s_cmp_eq_u32 %0, 0\n\ts_cbranch_scc1 1f\n\ts_setprio %1\n1:" ::"s"(on), "i"(P) : "scc");
}

// Issue priority that falls with a wavefront's progress through its NG
// groups (3 in the first quarter, 0 in the last), when `on`: with the whole
// grid resident, the wavefronts sharing a SIMD then finish together instead
// of oldest first (the hardware's order), which would leave the last-staged
// one decoding alone at the end.  With several generations of wavefronts it
// would hold back the ones about to free their slots, so the host passes 0.
// Decode-only kernels keep the hardware's order: there the staggered ends
// overlap each wavefront's output stores with the others' decoding.  g must
// fold to a constant (fully unrolled loops).
template <int NG>
LW_DEV void lw_ramp(int on, int g)
{
    if (g == 0) lw_progress_priority<3>(on);
    if (g == NG / 4) lw_progress_priority<2>(on);
    if (g == NG / 2) lw_progress_priority<1>(on);
    if (g == 3 * NG / 4) lw_progress_priority<0>(on);
}

// Bit of lane stream l of tile t where bundle part k begins (0 <= k <
// 2 * a.parts; parts 0 .. a.parts-1 cover the first tile row, the rest the
// second; part 0 begins at bit 0).  The load is unconditional (index
// clamped), so it can be issued with the kernel's other prologue loads.
LW_DEV uint32_t lw_part_start(const KArgs &a, int64_t t, int l, int k)
{
    const size_t np1 = (size_t)(2 * a.parts - 1);
    const uint32_t v = a.split[((size_t)t * np1 + (size_t)(k > 0 ? k - 1 : 0)) * 32 + (size_t)l];
    return k > 0 ? v : 0u;
}

// Set up a lane's decoder on its staged tile.  Returns false (the kernel must
// then produce nothing) unless the LDS base is 512-byte aligned (the shift
// amounts s = A >> 1 then carry a bias lb/2 + PBASE/2 that is a multiple of
// 64, which both the 32-bit shifts and the 64-bit window offset need, the
// low byte of a compact table's A is its byte-table selector, and that of
// the sparse plan's A >> 1) and low enough that the compact selector's
// second byte stays a 0xFF selector and its upper bytes stay zero.
LW_DEV bool lw_lane_init(LaneDec &d, uint8_t *lds, const uint32_t *slots, int l, const KArgs &a)
{
    const uint32_t lb = (uint32_t)(size_t)lds;
    d.wref = (uint32_t)(size_t)(slots + l) - 4u;
    d.un = ~31u;
    d.k = a.sad_k + lb;
    d.lut_lo = a.lut_lo;
    d.xk[0] = a.xk[0];
    d.xk[1] = a.xk[1];
    // Wave-uniform operands that a VOP3 instruction takes beside a scalar
    // one (it may read a single scalar register) are held in vector
    // registers, set once here, so the decode loops make no copy per group
    // (a VALU instruction that reads a scalar register also issues at the
    // slower rate on gfx950).
    asm volatile("" : "+v"(d.k), "+v"(d.lut_lo), "+v"(d.xk[0]), "+v"(d.xk[1]));
    d.ubias = 4u * (lb / 2u + LW_PBASE / 2u);
    return (lb & 511u) == 0 && lb + LW_CSEL < 0xFF00u;
}

// The exchange tree of the split-column reduction.  When a row band's
// columns are split over several workgroups (column groups), their sums are
// combined in a binary tree over the groups (a node without a sibling at
// some level passes its value up unchanged).  For each output, the two
// members of a pair meet in one slot of the bundle's workspace, which holds
// 0 when empty: each swaps its value into the slot with one device-scope
// atomic exchange.  The one that gets 0 back arrives first and is done; the
// other gets its partner's value, empties the slot again and carries the sum
// one level up.  The single atomic read-modify-write on the slot is the only
// synchronisation, so no thread ever waits for another, and every slot is
// empty again when the call ends (both members of every pair always come).
// Floating-point addition is commutative, so each pair's sum, and the whole
// tree's, does not depend on which member arrives first: the result is
// deterministic.  A value of +0.0 travels as -0.0 (the empty slot's bits are
// those of +0.0), so an output whose sum is zero may be written as -0.0.
//
// This thread's outputs v[k] (at their indices at[k] in y, -1 for none)
// enter as leaf `node` of a tree over n leaves and go up level by level,
// their exchanges in flight at once: ceil(log2(n)) round trips to the
// coherence point.  On return at[k] is -1 where this thread arrived first at
// some pair (its partner carries the sum on); the outputs left in at[] hold
// their complete sums.
template <int KMAX>
LW_DEV void lw_tree_combine(const KArgs &a, int node, int n, float (&v)[KMAX], int64_t (&at)[KMAX])
{
    uint32_t *slots = reinterpret_cast<uint32_t *>(a.part);
    const size_t stride = (size_t)LW_BATCH_MAX * (size_t)a.rows;   // one slot: [LW_BATCH_MAX][rows]
    int base = 0;
    while (n > 1) {
        if ((node ^ 1) < n) {
            uint32_t *slot = slots + (size_t)(base + (node >> 1)) * stride;
            uint32_t mine[KMAX], other[KMAX];
#pragma unroll
            for (int k = 0; k < KMAX; k++) {
                mine[k] = __builtin_bit_cast(uint32_t, v[k]);
                if (mine[k] == 0u) mine[k] = 0x80000000u;
                other[k] = at[k] >= 0 ? __hip_atomic_exchange(slot + at[k], mine[k], __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT)
                                      : 0u;
            }
#pragma unroll
            for (int k = 0; k < KMAX; k++) {
                if (at[k] < 0) continue;
                if (other[k] == 0u) {
                    at[k] = -1;                          // first of the pair: the partner carries on
                } else {
                    __hip_atomic_store(slot + at[k], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    v[k] = __builtin_bit_cast(float, mine[k]) + __builtin_bit_cast(float, other[k]);
                }
            }
        }
        base += n >> 1;                                  // pair slots used at this level
        node >>= 1;
        n = (n + 1) >> 1;
    }
}

// Sum the per-wave partials of the workgroup's ROWS rows (red[wave][b][row],
// RS floats between consecutive (wave, b) runs) and write y, or, when the
// row band's columns are split over a.groups workgroups, combine the groups'
// sums in the exchange tree (leaf g).
template <int BATCH, int ROWS = 128, int RS = ROWS>
LW_DEV void lw_finish_rows(const KArgs &a, const float *red, int64_t row0, int g, int waves)
{
    constexpr int KMAX = (BATCH * ROWS + 255) / 256;   // outputs per thread (workgroups have at least 256 threads)
    float v[KMAX];
    int64_t at[KMAX];                                    // the output's index in y, or -1
#pragma unroll
    for (int k = 0; k < KMAX; k++) {
        const int i = (int)threadIdx.x + k * (int)blockDim.x;
        const int b = i / ROWS, row = i % ROWS;
        const bool ok = i < BATCH * ROWS && b < a.batch && row0 + row < a.rows;
        float s = 0.f;
        if (ok)
            for (int w = 0; w < waves; w++) s += red[(w * BATCH + b) * RS + row];
        v[k] = s;
        at[k] = ok ? (int64_t)b * a.rows + row0 + row : -1;
    }
    if (a.groups > 1) lw_tree_combine<KMAX>(a, g, a.groups, v, at);
#pragma unroll
    for (int k = 0; k < KMAX; k++)
        if (at[k] >= 0) a.y[at[k]] = v[k];
}

// Finish of the balanced layouts (fused_q.hip, mfma.hip): workgroup k holds
// tiles [kU, kU + U) in row-major order, U = 4K + 2, with wavefronts 0 ..
// 4K-1 on tiles 0 .. 4K-1 and wavefronts 4K + i on tile 4K + i/2.  Its tiles
// cover row band rb0 from slot 0 and, when the band ends inside, band rb0 + 1
// from slot jb.  Each (band, batch row, row) output sums red[wave][b][row]
// (RS floats between (wave, b) runs) over the band's wavefronts in wavefront
// order, then meets the other workgroups holding the band's tiles in the
// exchange tree (leaf = k - the band's first workgroup).  A thread's KMAX
// outputs are consecutive, so they share a band.
template <int BATCH, int RS, int K>
LW_DEV void lw_finish_balanced(const KArgs &a, const float *red)
{
    constexpr int U = 4 * K + 2, WPG = 4 * K + 4, NOUT = 2 * BATCH * 64;
    constexpr int KMIN = (NOUT + 64 * WPG - 1) / (64 * WPG);   // outputs per thread, rounded up to a power of two
    constexpr int KMAX = KMIN <= 1 ? 1 : KMIN <= 2 ? 2 : KMIN <= 4 ? 4 : 8;
    static_assert((BATCH * 64) % KMAX == 0 && 64 * WPG * KMAX >= NOUT, "a thread's outputs share a band");
    const int64_t T0 = (int64_t)blockIdx.x * U;
    const int rb0 = (int)(T0 / a.n_cb);
    const int jb = (int)((int64_t)(rb0 + 1) * a.n_cb - T0);   // first slot of the next band (>= U: none)
    const int s = (int)(threadIdx.x * KMAX) / (BATCH * 64);   // band of this thread's outputs: rb0 + s
    const int band = rb0 + s;
    float v[KMAX];
    int64_t at[KMAX];
    bool any = false;
#pragma unroll
    for (int k = 0; k < KMAX; k++) {
        const int i = (int)threadIdx.x * KMAX + k;
        const int b = (i / 64) % BATCH, r = i % 64;
        const bool ok = i < NOUT && b < a.batch && (s == 0 || jb < U) && band < a.n_rb;
        float sum = 0.f;
        if (ok)
            for (int w = 0; w < WPG; w++) {
                const int jw = w < 4 * K ? w : 4 * K + ((w - 4 * K) >> 1);
                if ((jw >= jb) == (s == 1)) sum += red[(w * BATCH + b) * RS + r];
            }
        v[k] = sum;
        at[k] = ok ? (int64_t)b * a.rows + (int64_t)band * 64 + r : -1;
        any = any || ok;
    }
    if (any) {
        // the workgroups holding this band's tiles
        const int64_t f = (int64_t)band * a.n_cb / U, e = ((int64_t)band * a.n_cb + a.n_cb - 1) / U;
        if (e > f) lw_tree_combine<KMAX>(a, (int)(blockIdx.x - f), (int)(e - f + 1), v, at);
    }
#pragma unroll
    for (int k = 0; k < KMAX; k++)
        if (at[k] >= 0) a.y[at[k]] = v[k];
}

#endif
