// bundle.cpp -- host-side bundle builder of liblw ("LazyWeights: Decode-on-
// Demand Edge LLMs", section "2 . Code them"; bf16 variant after "Unweight",
// "The exponent's exploitable redundancy").
//
// A bundle is a flat image (lw_internal.h) holding, for one matrix:
//   - one length-limited (<= 11 bit) canonical Huffman table,
//   - the lane words of every 64x256 tile: 32 lanes, each carrying two
//     adjacent rows as its own MSB-first bit stream cut into 32-bit words,
//     the lanes' words interleaved (word j of lane l at 32j + l) and zero-padded to the tile's
//     longest lane, plus a word offset per tile,
//   - the raw per-super-block scales (Q4/Q6), or the raw sign+mantissa bytes,
//     exponent palette and verbatim segments (bf16),
//   - tables derived for the GPU kernels and a zeroed device workspace.
// Choices the pages leave open (tie-breaks, bit order, lane rows, pair order)
// are the ones listed in the design notes; they make the image reproducible.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "lw_internal.h"

struct lw_bundle {
    std::vector<uint8_t> image;
};

// ----------------------------------------------------------------- errors
static thread_local std::string g_err;

lw_status lw_fail(lw_status s, const std::string &msg)
{
    g_err = msg;
    return s;
}

extern "C" const char *lw_last_error(void) { return g_err.c_str(); }

extern "C" const char *lw_status_str(lw_status s)
{
    switch (s) {
    case LW_OK: return "ok";
    case LW_E_ARG: return "invalid argument";
    case LW_E_SHAPE: return "shape not a multiple of 64x256";
    case LW_E_TABLE: return "invalid code table";
    case LW_E_FORMAT: return "corrupt bundle";
    case LW_E_NOMEM: return "out of host memory";
    case LW_E_DEVICE: return "HIP error";
    case LW_E_UNSUPPORTED: return "unsupported";
    }
    return "unknown status";
}

// ----------------------------------------------------------------- helpers
static int worker_count()
{
    unsigned n = std::thread::hardware_concurrency();
    if (n == 0) n = 4;
    return (int)std::min(n, 16u);
}

template <class F>
static void parallel_for(int64_t n, F f)
{
    int nt = (int)std::min<int64_t>(worker_count(), std::max<int64_t>(n, 1));
    if (nt <= 1) {
        for (int64_t i = 0; i < n; i++) f(i);
        return;
    }
    std::atomic<int64_t> next(0);
    std::vector<std::thread> th;
    for (int t = 0; t < nt; t++)
        th.emplace_back([&]() {
            for (;;) {
                int64_t i = next.fetch_add(1);
                if (i >= n) break;
                f(i);
            }
        });
    for (auto &x : th) x.join();
}

// Code lengths of the format: the optimal prefix code whose lengths do not
// exceed 11 bits ("2 . Code them": a length-limited Huffman table with
// 11-bit codes), found by package-merge (Larmore and Hirschberg's
// coin-collector method).  Each symbol with a nonzero count is a coin of
// every denomination 2^-1 .. 2^-11; packages are formed level by level from
// the smallest denominations up, and the cheapest 2n - 2 items of the last
// level give every symbol's length as the number of items it appears in.
// Ties are broken so that the result is reproducible: leaves ordered by
// (count, symbol), a level's items paired in list order, and a leaf placed
// before a package of equal weight.
//
// Here the items live in one arena: a leaf refers to its symbol, a package
// to its two children, and a symbol's length is counted by walking the
// chosen items down to their leaves.
namespace {
struct PmItem {
    uint64_t w;
    int32_t a, b;                  // leaf: a = symbol, b = -1; package: the two child items
};
}

static bool package_merge_lengths(int n_alpha, const uint64_t *counts, uint8_t *lens)
{
    std::vector<int> leaves;
    for (int s = 0; s < n_alpha; s++) {
        lens[s] = 0;
        if (counts[s]) leaves.push_back(s);
    }
    const int n = (int)leaves.size();
    if (n == 0) return true;
    if (n == 1) {
        lens[leaves[0]] = 1;
        return true;
    }
    if (n > (1 << LW_MAXLEN)) return false;
    std::stable_sort(leaves.begin(), leaves.end(), [&](int x, int y) { return counts[x] < counts[y]; });
    std::vector<PmItem> arena;
    arena.reserve((size_t)n * (LW_MAXLEN + 1) * 2);
    std::vector<int32_t> leaf_item(n);
    for (int i = 0; i < n; i++) {
        leaf_item[i] = (int32_t)arena.size();
        arena.push_back(PmItem{counts[leaves[i]], leaves[i], -1});
    }
    std::vector<int32_t> level(leaf_item), next;
    for (int depth = 1; depth < LW_MAXLEN; depth++) {
        // packages of adjacent items of this level, in order
        std::vector<int32_t> pk;
        for (size_t k = 0; k + 1 < level.size(); k += 2) {
            pk.push_back((int32_t)arena.size());
            arena.push_back(PmItem{arena[level[k]].w + arena[level[k + 1]].w, level[k], level[k + 1]});
        }
        // the next level: the leaves and these packages by weight, a leaf first on ties
        next.clear();
        size_t i = 0, j = 0;
        while (i < leaf_item.size() || j < pk.size()) {
            const bool leaf = j == pk.size() || (i < leaf_item.size() && arena[leaf_item[i]].w <= arena[pk[j]].w);
            next.push_back(leaf ? leaf_item[i++] : pk[j++]);
        }
        level.swap(next);
    }
    // walk the first 2n - 2 items down to their leaves
    std::vector<int32_t> stack;
    std::vector<uint32_t> depthcount(n_alpha, 0);
    for (int k = 0; k < 2 * n - 2 && k < (int)level.size(); k++) {
        stack.push_back(level[k]);
        while (!stack.empty()) {
            const PmItem it = arena[stack.back()];
            stack.pop_back();
            if (it.b < 0) {
                depthcount[it.a]++;
            } else {
                stack.push_back(it.a);
                stack.push_back(it.b);
            }
        }
    }
    for (int s = 0; s < n_alpha; s++) {
        if (depthcount[s] > LW_MAXLEN) return false;
        lens[s] = (uint8_t)depthcount[s];
    }
    return true;
}

// The compact code (an opt-in of lw_bundle_build_q_compact and
// lw_bundle_build_bf16_compact, not the format's default): the cheapest
// prefix code with lengths <= 11 that uses at most four distinct lengths, the
// three shorter of them <= 8.  A lane then finds a code's length with one
// pair of byte-sum comparisons of the top 8 peek bits and the shift from a
// four-entry byte table (lane_decode.hpp).  Against the optimal code this
// costs bits: +0.6 % on the 4-bit pair histogram of the up projection,
// +2.2 % on the sharper histogram of the down projection.
//
// Symbols with a nonzero count are ranked by (count desc, symbol asc); a
// length set a < b < c <= 8, c < d <= 11 takes the first n1 ranks at length
// a, the next n2 at b, then n3 at c and the rest at d, with n3 as large as
// the Kraft sum allows (moving a rank from d to c only saves bits).  Every
// (a, b, c, d, n1, n2) is tried in ascending lexicographic order and the
// first strictly cheapest total wins; a lone symbol gets length 1.
static bool compact_lengths(int n_alpha, const uint64_t *counts, uint8_t *lens)
{
    std::vector<int> rank;
    for (int s = 0; s < n_alpha; s++) {
        lens[s] = 0;
        if (counts[s]) rank.push_back(s);
    }
    const int n = (int)rank.size();
    if (n == 0) return true;
    if (n == 1) {
        lens[rank[0]] = 1;
        return true;
    }
    if (n > 256) return false;
    std::stable_sort(rank.begin(), rank.end(), [&](int x, int y) { return counts[x] > counts[y]; });
    std::vector<uint64_t> pre(n + 1, 0);                    // pre[k]: total count of the first k ranks
    for (int i = 0; i < n; i++) pre[i + 1] = pre[i] + counts[rank[i]];
    const int64_t KR = 1 << LW_MAXLEN;                      // Kraft budget in units of 2^-11
    uint64_t best = ~(uint64_t)0;
    int bl[4] = {0, 0, 0, 0}, bn[3] = {0, 0, 0};
    for (int a = 1; a <= 8; a++)
        for (int b = a + 1; b <= 8; b++)
            for (int c = b + 1; c <= 8; c++)
                for (int d = c + 1; d <= LW_MAXLEN; d++) {
                    const int64_t ua = KR >> a, ub = KR >> b, uc = KR >> c, ud = KR >> d;
                    for (int n1 = 0; n1 <= n && n1 * ua <= KR; n1++)
                        for (int n2 = 0; n1 + n2 <= n && n1 * ua + n2 * ub <= KR; n2++) {
                            const int64_t rest = n - n1 - n2;
                            const int64_t room = KR - n1 * ua - n2 * ub;
                            if (rest * ud > room) continue;
                            const int64_t n3 = std::min<int64_t>(rest, (room - rest * ud) / (uc - ud));
                            const int k1 = n1, k2 = n1 + n2, k3 = k2 + (int)n3;
                            const uint64_t cost = (uint64_t)a * pre[k1] + (uint64_t)b * (pre[k2] - pre[k1]) +
                                                  (uint64_t)c * (pre[k3] - pre[k2]) + (uint64_t)d * (pre[n] - pre[k3]);
                            if (cost < best) {
                                best = cost;
                                bl[0] = a, bl[1] = b, bl[2] = c, bl[3] = d;
                                bn[0] = k1, bn[1] = k2, bn[2] = k3;
                            }
                        }
                }
    for (int i = 0; i < n; i++) lens[rank[i]] = (uint8_t)(i < bn[0] ? bl[0] : i < bn[1] ? bl[1] : i < bn[2] ? bl[2] : bl[3]);
    return true;
}

// Canonical code in the RFC 1951 (section 3.2.2) manner, and the decoder
// arrays of "3 . Decode on demand": per length L, count, first code,
// limit = (first + count) << (11 - L), and offset into the length-sorted
// symbol table.
static int canonical_table(int n_alpha, const uint8_t *lens, uint16_t *codes, lw_table *t)
{
    std::memset(t, 0, sizeof(*t));
    for (int s = 0; s < n_alpha; s++) {
        if (lens[s] > LW_MAXLEN) return -1;
        if (lens[s]) t->count[lens[s]]++;
    }
    uint32_t next[LW_MAXLEN + 2];
    uint32_t code = 0;
    for (int L = 1; L <= LW_MAXLEN; L++) {
        code = (code + t->count[L - 1]) << 1;
        next[L] = code;
        t->first[L] = (uint16_t)code;
    }
    uint32_t acc = 0;
    for (int L = 1; L <= LW_MAXLEN; L++) {
        t->offset[L] = (uint16_t)acc;
        acc += t->count[L];
        t->limit[L] = (uint16_t)(((uint32_t)t->first[L] + t->count[L]) << (LW_MAXLEN - L));
    }
    uint32_t fill[LW_MAXLEN + 2];
    for (int L = 1; L <= LW_MAXLEN; L++) fill[L] = t->offset[L];
    for (int s = 0; s < n_alpha; s++) {
        codes[s] = 0;
        if (!lens[s]) continue;
        codes[s] = (uint16_t)next[lens[s]]++;
        t->sym_sorted[fill[lens[s]]++] = (uint16_t)s;
    }
    return (int)acc;
}

// Bit writer into one lane of an interleaved tile block.
struct LaneWriter {
    uint32_t *blk;
    int lane;
    uint64_t acc = 0;   // pending bits, right-aligned
    int nacc = 0;
    int64_t word = 0;
    uint64_t bits() const { return 32u * (uint64_t)word + (uint64_t)nacc; }
    void put(uint32_t code, int len)
    {
        acc = (acc << len) | code;
        nacc += len;
        if (nacc >= 32) {
            nacc -= 32;
            blk[32 * word + lane] = (uint32_t)(acc >> nacc);
            word++;
            acc &= (nacc ? ((1ull << nacc) - 1) : 0);
        }
    }
    void flush()
    {
        if (nacc) blk[32 * word + lane] = (uint32_t)(acc << (32 - nacc));
    }
};

struct Shape {
    int64_t rows, cols, n_rb, n_cb, n_tiles;
};

// Layout of a new image.  Returns the header with offsets and sizes filled.
static lw_image_header plan_image(int kind, const Shape &sh, int64_t n_words, int64_t n_verb, int parts)
{
    lw_image_header h;
    std::memset(&h, 0, sizeof(h));
    h.magic = LW_MAGIC;
    h.version = LW_VERSION;
    h.kind = kind;
    h.bits = kind == LW_Q4_PAIR ? 4 : (kind == LW_Q6_SINGLE ? 6 : 16);
    h.rows = sh.rows;
    h.cols = sh.cols;
    h.n_tiles = sh.n_tiles;
    h.n_rb = (int32_t)sh.n_rb;
    h.n_cb = (int32_t)sh.n_cb;
    h.spl = kind == LW_Q4_PAIR ? 256 : 512;
    h.parts = parts;
    h.work_groups = lw_work_groups(sh.n_cb, parts);
    h.n_verbatim = n_verb;
    uint64_t bytes[LW_REG_COUNT] = {0};
    bytes[LW_REG_TABLE] = sizeof(lw_table);
    bytes[LW_REG_GPUTAB] = sizeof(lw_gputab);
    bytes[LW_REG_TILE_OFF] = 4u * (uint64_t)(sh.n_tiles + 1);
    bytes[LW_REG_WORDS] = 4u * (uint64_t)n_words;
    bytes[LW_REG_SPLIT] = 2u * LW_LANES * (uint64_t)sh.n_tiles * (uint64_t)(2 * parts - 1);
    if (kind == LW_BF16_EXP) {
        bytes[LW_REG_PALETTE] = 16;
        bytes[LW_REG_SM] = 4u * 4096u * (uint64_t)sh.n_tiles;
        bytes[LW_REG_VB_BITS] = 32u * (uint64_t)sh.n_tiles;
        bytes[LW_REG_VB_START] = 4u * (uint64_t)(sh.n_tiles + 1);
        bytes[LW_REG_VERBATIM] = 128u * (uint64_t)n_verb;
    } else {
        bytes[LW_REG_DM] = 4u * 64u * (uint64_t)sh.n_tiles;
    }
    // the pair slots of the split-column reduction
    bytes[LW_REG_WORK] = lw_work_bytes(h.work_groups, sh.rows);
    uint64_t pos = LW_HEADER_BYTES;
    for (int r = 0; r < LW_REG_COUNT; r++) {
        h.off[r] = bytes[r] ? pos : 0;
        h.bytes[r] = bytes[r];
        pos = lw_align_up(pos + bytes[r]);
    }
    h.coded_bytes = bytes[LW_REG_WORDS] + bytes[LW_REG_TILE_OFF] + bytes[LW_REG_SPLIT] + bytes[LW_REG_TABLE] +
                    bytes[LW_REG_DM] + bytes[LW_REG_SM] + bytes[LW_REG_VB_BITS] +
                    bytes[LW_REG_VB_START] + bytes[LW_REG_VERBATIM] + bytes[LW_REG_PALETTE];
    h.twin_bytes = kind == LW_BF16_EXP
        ? 2u * (uint64_t)sh.rows * (uint64_t)sh.cols
        : (uint64_t)sh.rows * (uint64_t)sh.cols * (uint64_t)h.bits / 8u +
              (uint64_t)sh.rows * (uint64_t)(sh.cols / 256) * 4u;
    return h;
}

template <class T>
static T *region(std::vector<uint8_t> &img, const lw_image_header &h, int r)
{
    return reinterpret_cast<T *>(img.data() + h.off[r]);
}

// fp16 bit pattern of a small non-negative integer (exact for v < 2048).
static uint32_t small_int_half(uint32_t v)
{
    if (v == 0) return 0;
    int e = 31 - __builtin_clz(v);
    return (uint32_t)((e + 15) << 10) | ((v << (10 - e)) & 0x3FFu);
}

// Derived tables for the kernels (payload per canonical index, limits
// left-justified to a 32-bit window, length and base per comparison count).
static void fill_gputab(int kind, const lw_table &t, const uint8_t *palette, lw_image_header &h,
                        lw_gputab *g)
{
    std::memset(g, 0, sizeof(*g));
    int lmin = 0, lmax = 0;
    for (int L = 1; L <= LW_MAXLEN; L++)
        if (t.count[L]) {
            if (!lmin) lmin = L;
            lmax = L;
        }
    h.min_len = lmin;
    h.max_len = lmax;
    for (int i = 0; i < 16; i++) g->limlj[i] = 0xFFFFFFFFu;
    for (int L = lmin; L < lmax; L++) g->limlj[L - lmin] = (uint32_t)t.limit[L] << 21;
    for (int r = 0; lmin && r <= lmax - lmin; r++) {
        int L = lmin + r;
        g->len[r] = (uint32_t)L;
        g->base[r] = (int32_t)t.offset[L] - (int32_t)t.first[L];
    }
    lw_make_plan(t, lmin, lmax, g->plan);
    for (int i = 0; i < h.n_sym; i++) {
        uint32_t s = t.sym_sorted[i];
        g->symval[i] = s;
        if (kind == LW_Q4_PAIR) {
            g->payload[i] = small_int_half(s & 15) | (small_int_half(s >> 4) << 16);
        } else if (kind == LW_Q6_SINGLE) {
            g->payload[i] = small_int_half(s);
            g->payload_hi[i] = small_int_half(s) << 16;
        } else {
            uint32_t e = palette[s];
            g->payload[i] = e << 7;
            g->payload_hi[i] = e << 23;
        }
    }
}

// Residue packing of the limits of lengths L[0..n) into two SAD byte pairs:
// a limit c with c mod 8 = r compares floor((p + k)/8) with (c + k)/8,
// k = 8 - r, on a byte taken from the peek plus k << 21 (a saturating add),
// or with `sub` floor((p - r)/8) with (c - r)/8 on a byte taken from the
// peek minus r << 21 (saturating at 0; this form also takes limits above
// 2040, where (c + k)/8 would be 256, and needs c - r >= 8); the residue-0
// limits compare the top byte.  Residue limits of pair j sit in its top bytes
// (3, 2, ..), read from the peek plus k_j; the residue-0 limits fill bytes
// 0.. of pair 0, then of pair 1.  One residue: its limits split over both
// pairs, which share one register.  Unused lanes compare 0 with 0 and
// contribute nothing.  Writes c8, c8m1, xk and xsel of a and returns the
// number of residues besides 0 (0..2), or -1 when the limits do not fit.
static int pack_residues(const lw_table &t, const int *L, int n, lw_plan &a, bool sub)
{
    if (n > 8) return -1;
    int thr[8], zero[8], rl[2][8], nz = 0, nrl[2] = {0, 0}, rv[2] = {0, 0}, nres = 0;
    for (int i = 0; i < n; i++) {
        const uint32_t c = t.limit[L[i]];
        const int r = (int)(c & 7u);
        thr[i] = sub ? (int)((c - (uint32_t)r) >> 3) : (int)((c + (uint32_t)((8 - r) & 7)) >> 3);   // exact
        if (thr[i] < 1 || thr[i] > 255) return -1;
        if (!r) {
            zero[nz++] = i;
            continue;
        }
        int q = -1;
        for (int j = 0; j < nres; j++)
            if (rv[j] == r) q = j;
        if (q < 0) {
            if (nres == 2) return -1;
            q = nres;
            rv[nres++] = r;
        }
        rl[q][nrl[q]++] = i;
    }
    int pres[2] = {0, 0}, plist[2][8], pn[2] = {0, 0};
    if (nres == 1) {
        pres[0] = pres[1] = rv[0];
        for (int i = 0; i < nrl[0]; i++) {
            const int j = i & 1;
            plist[j][pn[j]++] = rl[0][i];
        }
    } else if (nres == 2) {
        for (int j = 0; j < 2; j++) {
            pres[j] = rv[j];
            for (int i = 0; i < nrl[j]; i++) plist[j][pn[j]++] = rl[j][i];
        }
    }
    const int extra = std::max(pn[0], pn[1]);
    if (extra > 4 || nz > 2 * (4 - extra)) return -1;
    a.c8[0] = a.c8[1] = a.c8m1[0] = a.c8m1[1] = 0;
    for (int j = 0; j < 2; j++)
        for (int i = 0; i < pn[j]; i++) {
            const int b = 3 - i;
            a.c8[j] |= (uint32_t)thr[plist[j][i]] << (8 * b);
            a.c8m1[j] |= (uint32_t)(thr[plist[j][i]] - 1) << (8 * b);
        }
    for (int i = 0; i < nz; i++) {
        const int j = i / (4 - extra), b = i % (4 - extra);
        a.c8[j] |= (uint32_t)thr[zero[i]] << (8 * b);
        a.c8m1[j] |= (uint32_t)(thr[zero[i]] - 1) << (8 * b);
    }
    for (int j = 0; j < 2; j++) {
        const int k = sub ? pres[j] : (8 - pres[j]) & 7;
        a.xk[j] = (uint32_t)k << 21;
        uint32_t sel = 0;
        for (int b = 0; b < 4; b++) sel |= (k && b >= 4 - extra ? 7u : 3u) << (8 * b);
        a.xsel[j] = sel;
    }
    return nres;
}

// Limit comparisons packed for the SAD counting of lane_decode.hpp.
// Compact tables (at most four used lengths, the three shorter <= 8): the
// limits of the used lengths but the longest, in byte lanes (top 8 peek bits
// against limit/8), the count indexing the used lengths.  Other tables
// compare every length min_len .. max_len-1 (an absent length repeats the
// previous limit), so the length is min_len + count:
//   - up to eight limits whose residues mod 8 take at most two values besides
//     0 go to two SAD byte pairs (residue plans, pack_residues);
//   - when these do not fit but the used lengths but the longest (at most
//     seven) do, with at most one residue in the subtracting form, the
//     sparse plan compares only those, and the count r indexes the used
//     lengths through a byte table (the length of count r in byte 7 - r);
//   - anything else takes the general plan (lengths <= 8 in byte lanes, 9 and
//     10 in 16-bit lanes against the top 16 window bits).
void lw_make_plan(const lw_table &t, int min_len, int max_len, lw_plan &a)
{
    std::memset(&a, 0, sizeof(a));
    a.c8[0] = a.c8[1] = a.c8m1[0] = a.c8m1[1] = 0;
    a.c16 = a.c16m1 = 0;
    a.xsel[0] = a.xsel[1] = 0x03030303u;
    a.xk[0] = a.xk[1] = 0;
    a.lut_lo = a.lut_hi = 0;
    a.cbase[0] = a.cbase[1] = a.cbase[2] = a.cbase[3] = 0;
    a.ncmp = 0;
    int used[LW_MAXLEN + 1], nu = 0;
    for (int L = 1; L <= LW_MAXLEN; L++)
        if (t.count[L]) used[nu++] = L;
    if (nu >= 1 && nu <= 4 && (nu == 1 || used[nu - 2] <= 8)) {
        uint64_t lut = 0x00FF00FF00FF00FFull;   // even bytes 0xFF: what the selector's zero upper bytes pick
        for (int r = 0; r < nu; r++) {
            const int L = used[r];
            lut |= (uint64_t)((256 - L) & 0xFF) << (8 * (7 - 2 * r));
            a.cbase[r] = (int32_t)t.offset[L] - (int32_t)t.first[L];
            if (r < nu - 1) {
                const uint32_t c = (uint32_t)t.limit[L] >> 3;
                a.c8[0] |= c << (8 * r);
                a.c8m1[0] |= (c - 1) << (8 * r);
            }
        }
        a.lut_lo = (uint32_t)lut;
        a.lut_hi = (uint32_t)(lut >> 32);
        a.ncmp = nu - 1;
        a.sad_k = LW_PLAN_CSEL - (uint32_t)(nu - 1);
        a.plan = LW_P_COMPACT;
        return;
    }
    const int n = max_len - min_len;          // comparisons: lengths min_len .. max_len - 1
    int dense[LW_MAXLEN + 1];
    for (int i = 0; i < n; i++) dense[i] = min_len + i;
    a.sad_k = LW_PLAN_PBASE - 2u * (uint32_t)min_len - (uint32_t)n;   // residue and general plans
    const int nres = pack_residues(t, dense, n, a, false);
    if (nres >= 0) {
        a.plan = nres == 0 ? LW_P_R2 : nres == 1 ? LW_P_R2K : LW_P_R2X2;
        return;
    }
    if (nu <= 8 && nu < n + 1) {
        const int sres = pack_residues(t, used, nu - 1, a, true);
        if (sres == 0 || sres == 1) {
            uint64_t lut = 0;
            for (int r = 0; r < nu; r++) lut |= (uint64_t)((256 - used[r]) & 0xFF) << (8 * (7 - r));
            a.lut_lo = (uint32_t)lut;
            a.lut_hi = (uint32_t)(lut >> 32);
            a.ncmp = nu - 1;
            a.sad_k = LW_PLAN_SBASE - (uint32_t)(nu - 1);
            a.plan = LW_P_S2K;
            return;
        }
    }
    a.xsel[0] = a.xsel[1] = 0x03030303u;
    a.xk[0] = a.xk[1] = 0;
    a.c8[0] = a.c8[1] = a.c8m1[0] = a.c8m1[1] = 0;
    int l8[8], l16[2], n8 = 0, n16 = 0;
    for (int L = min_len; L < max_len; L++) {
        if (L <= 8) l8[n8++] = L;
        else l16[n16++] = L;
    }
    for (int i = 0; i < n8; i++) {
        const uint32_t c = (uint32_t)t.limit[l8[i]] >> 3;
        a.c8[i / 4] |= c << (8 * (i % 4));
        a.c8m1[i / 4] |= (c - 1) << (8 * (i % 4));
    }
    for (int i = 0; i < n16; i++) {
        const uint32_t c = (uint32_t)t.limit[l16[i]] << 5;
        a.c16 |= c << (16 * i);
        a.c16m1 |= (c - 1) << (16 * i);
    }
    a.plan = LW_P_GEN;
}

// Encode every tile of a symbol source.  sym(t, l, k) gives symbol k of lane
// l of tile t.  Two passes: lane bit counts (for the tile sizes), then words
// and the part starts: with P = h->parts, lane stream l of tile t is 2P parts
// of spl/(2P) symbols (P per tile row), and split[(t*(2P-1) + k-1)*32 + l]
// is the bit where part k >= 1 begins.
template <class SymFn>
static void encode_tiles(const Shape &sh, int spl, const uint8_t *lens, const uint16_t *codes,
                         SymFn sym, std::vector<uint32_t> &tile_off, int32_t &max_words,
                         std::vector<uint8_t> *img, const lw_image_header *h)
{
    if (!img) {
        std::vector<uint32_t> wt(sh.n_tiles);
        parallel_for(sh.n_tiles, [&](int64_t t) {
            uint32_t wmax = 0;
            for (int l = 0; l < LW_LANES; l++) {
                uint64_t bits = 0;
                for (int k = 0; k < spl; k++) bits += lens[sym(t, l, k)];
                wmax = std::max<uint32_t>(wmax, (uint32_t)((bits + 31) / 32));
            }
            wt[t] = wmax;
        });
        tile_off.assign(sh.n_tiles + 1, 0);
        uint64_t pos = 0;
        max_words = 0;
        for (int64_t t = 0; t < sh.n_tiles; t++) {
            tile_off[t] = (uint32_t)pos;
            pos += 32u * wt[t];
            max_words = std::max<int32_t>(max_words, (int32_t)wt[t]);
        }
        tile_off[sh.n_tiles] = (uint32_t)pos;
        return;
    }
    uint32_t *words = region<uint32_t>(*img, *h, LW_REG_WORDS);
    uint16_t *split = region<uint16_t>(*img, *h, LW_REG_SPLIT);
    const int nparts = 2 * h->parts, per = spl / nparts;
    parallel_for(sh.n_tiles, [&](int64_t t) {
        uint32_t *blk = words + tile_off[t];
        for (int l = 0; l < LW_LANES; l++) {
            LaneWriter w{blk, l};
            for (int k = 0; k < spl; k++) {
                if (k > 0 && k % per == 0)
                    split[(t * (nparts - 1) + k / per - 1) * LW_LANES + l] = (uint16_t)w.bits();
                int s = sym(t, l, k);
                w.put(codes[s], lens[s]);
            }
            w.flush();
        }
    });
}

static lw_status check_shape(int64_t rows, int64_t cols, Shape &sh)
{
    if (rows <= 0 || cols <= 0 || rows % LW_TILE_ROWS || cols % LW_TILE_COLS)
        return lw_fail(LW_E_SHAPE, "rows must be a positive multiple of 64 and cols of 256");
    if (rows * cols > ((int64_t)1 << 34))
        return lw_fail(LW_E_ARG, "matrix too large for 32-bit word offsets");
    sh.rows = rows;
    sh.cols = cols;
    sh.n_rb = rows / LW_TILE_ROWS;
    sh.n_cb = cols / LW_TILE_COLS;
    sh.n_tiles = sh.n_rb * sh.n_cb;
    return LW_OK;
}

// Parts per tile row: 0 picks the largest of 8, 4, 2, 1 that keeps the
// matrix within LW_PART_UNITS decoding units (tiles x parts); for 4- and
// 6-bit codes also 2 where the tiles are an odd multiple of 512 between
// LW_PART_UNITS / 2 and LW_PART_UNITS and a row band has more than 16 column
// blocks (10 or 14 tiles per CU of a 256-CU MI355X with no whole-row layout:
// the half-row starts let every SIMD carry the same work).  Else 1, 2, 4 or
// 8 as asked.
static lw_status choose_parts(const Shape &sh, int &parts, bool quantised)
{
    if (parts == 0) {
        parts = 8;
        while (parts > 1 && sh.n_tiles * parts > LW_PART_UNITS) parts /= 2;
        if (parts == 1 && quantised && sh.n_tiles > LW_PART_UNITS / 2 && sh.n_tiles <= LW_PART_UNITS &&
            sh.n_tiles % 512 == 0 && (sh.n_tiles / 512) % 2 == 1 && sh.n_cb > 16)
            parts = 2;
        return LW_OK;
    }
    if (parts != 1 && parts != 2 && parts != 4 && parts != 8) return lw_fail(LW_E_ARG, "parts must be 0, 1, 2, 4 or 8");
    return LW_OK;
}

static lw_status finish_table(int n_alpha, const std::vector<uint64_t> &hist, int code, uint8_t *lens,
                              uint16_t *codes, lw_table &tab, int &n_sym)
{
    const bool ok = code == LW_CODE_COMPACT ? compact_lengths(n_alpha, hist.data(), lens)
                                            : package_merge_lengths(n_alpha, hist.data(), lens);
    if (!ok) return lw_fail(LW_E_TABLE, "alphabet does not fit the code");
    n_sym = canonical_table(n_alpha, lens, codes, &tab);
    if (n_sym < 0) return lw_fail(LW_E_TABLE, "code length above 11");
    return LW_OK;
}

// Code lengths given by the caller: every symbol that occurs needs a length
// of 1..11, an absent one may have 0, and the lengths must satisfy Kraft's
// inequality (a prefix code exists).
static lw_status user_table(int n_alpha, const std::vector<uint64_t> &hist, const uint8_t *user, uint8_t *lens,
                            uint16_t *codes, lw_table &tab, int &n_sym)
{
    uint64_t kraft = 0;                              // in units of 2^-11
    for (int s = 0; s < n_alpha; s++) {
        lens[s] = user[s];
        if (lens[s] > LW_MAXLEN || (hist[s] && lens[s] == 0))
            return lw_fail(LW_E_TABLE, "a symbol that occurs needs a code length of 1..11");
        if (lens[s]) kraft += 1ull << (LW_MAXLEN - lens[s]);
    }
    if (kraft > (1ull << LW_MAXLEN)) return lw_fail(LW_E_TABLE, "code lengths violate the Kraft inequality");
    n_sym = canonical_table(n_alpha, lens, codes, &tab);
    if (n_sym < 0) return lw_fail(LW_E_TABLE, "code length above 11");
    return LW_OK;
}

static lw_status build_q(int kind, int64_t rows, int64_t cols, const uint8_t *q, const uint16_t *d,
                         const uint16_t *m, const uint8_t *user_lens, int code, int parts, lw_bundle **out)
{
    if (!out) return lw_fail(LW_E_ARG, "out is null");
    *out = nullptr;
    if (!q || !d || !m) return lw_fail(LW_E_ARG, "null input");
    if (kind != LW_Q4_PAIR && kind != LW_Q6_SINGLE) return lw_fail(LW_E_ARG, "kind must be Q4 or Q6");
    Shape sh;
    lw_status st = check_shape(rows, cols, sh);
    if (st) return st;
    if ((st = choose_parts(sh, parts, true))) return st;
    const int qmax = kind == LW_Q4_PAIR ? 15 : 63;
    const int n_alpha = kind == LW_Q4_PAIR ? 256 : 64;
    const int spl = kind == LW_Q4_PAIR ? 256 : 512;
    try {
        // histogram over the whole matrix (one table per matrix), per row band
        std::vector<std::vector<uint64_t>> part(sh.n_rb, std::vector<uint64_t>(n_alpha, 0));
        std::atomic<int> bad(0);
        parallel_for(sh.n_rb, [&](int64_t rb) {
            auto &hh = part[rb];
            for (int64_t r = rb * 64; r < rb * 64 + 64; r++) {
                const uint8_t *row = q + r * cols;
                if (kind == LW_Q4_PAIR) {
                    for (int64_t c = 0; c < cols; c += 2) {
                        if ((row[c] | row[c + 1]) > qmax) bad = 1;
                        hh[(row[c] | (row[c + 1] << 4)) & 255]++;
                    }
                } else {
                    for (int64_t c = 0; c < cols; c++) {
                        if (row[c] > qmax) bad = 1;
                        hh[row[c] & 63]++;
                    }
                }
            }
        });
        if (bad) return lw_fail(LW_E_ARG, "code out of range for the kind");
        std::vector<uint64_t> hist(n_alpha, 0);
        for (auto &hh : part)
            for (int s = 0; s < n_alpha; s++) hist[s] += hh[s];
        uint8_t lens[256];
        uint16_t codes[256];
        lw_table tab;
        int n_sym = 0;
        st = user_lens ? user_table(n_alpha, hist, user_lens, lens, codes, tab, n_sym)
                       : finish_table(n_alpha, hist, code, lens, codes, tab, n_sym);
        if (st) return st;

        auto sym = [&](int64_t t, int l, int k) -> int {
            int64_t rb = t / sh.n_cb, cb = t % sh.n_cb;
            int half = k >= spl / 2;
            int kk = k - half * (spl / 2);
            const uint8_t *row = q + (rb * 64 + 2 * l + half) * cols + cb * 256;
            if (kind == LW_Q4_PAIR) return row[2 * kk] | (row[2 * kk + 1] << 4);
            return row[kk];
        };
        std::vector<uint32_t> tile_off;
        int32_t max_words = 0;
        encode_tiles(sh, spl, lens, codes, sym, tile_off, max_words, nullptr, nullptr);
        lw_image_header h = plan_image(kind, sh, tile_off[sh.n_tiles], 0, parts);
        h.n_sym = n_sym;
        h.max_words = max_words;
        h.code = user_lens ? LW_CODE_LENS : code;
        std::unique_ptr<lw_bundle> b(new lw_bundle);
        uint64_t total = lw_align_up(h.off[LW_REG_WORK] + h.bytes[LW_REG_WORK]);
        for (int r = 0; r < LW_REG_COUNT; r++)
            if (h.bytes[r]) total = std::max<uint64_t>(total, lw_align_up(h.off[r] + h.bytes[r]));
        b->image.assign(total, 0);
        std::memcpy(region<uint32_t>(b->image, h, LW_REG_TILE_OFF), tile_off.data(), 4 * tile_off.size());
        *region<lw_table>(b->image, h, LW_REG_TABLE) = tab;
        fill_gputab(kind, tab, nullptr, h, region<lw_gputab>(b->image, h, LW_REG_GPUTAB));
        encode_tiles(sh, spl, lens, codes, sym, tile_off, max_words, &b->image, &h);
        uint32_t *dm = region<uint32_t>(b->image, h, LW_REG_DM);
        parallel_for(sh.n_rb, [&](int64_t rb) {
            for (int64_t cb = 0; cb < sh.n_cb; cb++)
                for (int i = 0; i < 64; i++) {
                    int64_t r = rb * 64 + i;
                    dm[(rb * sh.n_cb + cb) * 64 + i] =
                        (uint32_t)d[r * sh.n_cb + cb] | ((uint32_t)m[r * sh.n_cb + cb] << 16);
                }
        });
        std::memcpy(b->image.data(), &h, sizeof(h));
        *out = b.release();
        return LW_OK;
    } catch (const std::bad_alloc &) {
        return lw_fail(LW_E_NOMEM, "host allocation failed");
    }
}

extern "C" lw_status lw_bundle_build_q(int kind, int64_t rows, int64_t cols, const uint8_t *q,
                                       const uint16_t *d, const uint16_t *m, lw_bundle **out)
{
    return build_q(kind, rows, cols, q, d, m, nullptr, LW_CODE_HUFFMAN, 0, out);
}

extern "C" lw_status lw_bundle_build_q_compact(int kind, int64_t rows, int64_t cols, const uint8_t *q,
                                               const uint16_t *d, const uint16_t *m, lw_bundle **out)
{
    return build_q(kind, rows, cols, q, d, m, nullptr, LW_CODE_COMPACT, 0, out);
}

extern "C" lw_status lw_bundle_build_q_lens(int kind, int64_t rows, int64_t cols, const uint8_t *q,
                                            const uint16_t *d, const uint16_t *m, const uint8_t *lens,
                                            lw_bundle **out)
{
    if (!lens) {
        if (out) *out = nullptr;
        return lw_fail(LW_E_ARG, "lens is null");
    }
    return build_q(kind, rows, cols, q, d, m, lens, LW_CODE_LENS, 0, out);
}

// Options: the code (lens for LW_CODE_LENS) and the parts per tile row.
static lw_status check_opts(const lw_build_opts *o, lw_bundle **out)
{
    if (out) *out = nullptr;
    if (!o) return lw_fail(LW_E_ARG, "opts is null");
    if (o->code < LW_CODE_HUFFMAN || o->code > LW_CODE_LENS) return lw_fail(LW_E_ARG, "unknown code kind");
    if (o->code == LW_CODE_LENS && !o->lens) return lw_fail(LW_E_ARG, "lens is null");
    return LW_OK;
}

extern "C" lw_status lw_bundle_build_q_opts(int kind, int64_t rows, int64_t cols, const uint8_t *q,
                                            const uint16_t *d, const uint16_t *m, const lw_build_opts *opts,
                                            lw_bundle **out)
{
    lw_status st = check_opts(opts, out);
    if (st) return st;
    return build_q(kind, rows, cols, q, d, m, opts->code == LW_CODE_LENS ? opts->lens : nullptr, opts->code,
                   opts->parts, out);
}

static lw_status build_bf16(int64_t rows, int64_t cols, const uint16_t *w, int code, int parts, lw_bundle **out)
{
    if (!out) return lw_fail(LW_E_ARG, "out is null");
    *out = nullptr;
    if (!w) return lw_fail(LW_E_ARG, "null input");
    Shape sh;
    lw_status st = check_shape(rows, cols, sh);
    if (st) return st;
    if ((st = choose_parts(sh, parts, false))) return st;
    try {
        // exponent histogram -> palette: top 16 by (count desc, exponent asc)
        std::vector<std::vector<uint64_t>> part(sh.n_rb, std::vector<uint64_t>(256, 0));
        parallel_for(sh.n_rb, [&](int64_t rb) {
            for (int64_t i = rb * 64 * cols; i < (rb + 1) * 64 * cols; i++) part[rb][(w[i] >> 7) & 255]++;
        });
        uint64_t ecount[256] = {0};
        for (auto &p : part)
            for (int e = 0; e < 256; e++) ecount[e] += p[e];
        int order[256];
        for (int e = 0; e < 256; e++) order[e] = e;
        std::stable_sort(order, order + 256, [&](int a, int b) { return ecount[a] > ecount[b]; });
        uint8_t palette[16] = {0};
        int n_pal = 0;
        int8_t pidx[256];
        std::memset(pidx, -1, sizeof(pidx));
        for (int k = 0; k < 16 && ecount[order[k]]; k++) {
            palette[k] = (uint8_t)order[k];
            pidx[order[k]] = (int8_t)k;
            n_pal++;
        }
        // verbatim segments: any exponent outside the palette in a 64-weight run
        std::vector<uint32_t> vb_bits(sh.n_tiles * 8, 0), vb_start(sh.n_tiles + 1, 0);
        std::vector<uint32_t> tile_nv(sh.n_tiles, 0);
        parallel_for(sh.n_tiles, [&](int64_t t) {
            int64_t rb = t / sh.n_cb, cb = t % sh.n_cb;
            uint32_t nv = 0;
            for (int i = 0; i < 64; i++)
                for (int s = 0; s < 4; s++) {
                    const uint16_t *seg = w + (rb * 64 + i) * cols + cb * 256 + 64 * s;
                    bool outp = false;
                    for (int c = 0; c < 64; c++) outp |= pidx[(seg[c] >> 7) & 255] < 0;
                    if (outp) {
                        vb_bits[t * 8 + (4 * i + s) / 32] |= 1u << ((4 * i + s) % 32);
                        nv++;
                    }
                }
            tile_nv[t] = nv;
        });
        int64_t n_verb = 0;
        for (int64_t t = 0; t < sh.n_tiles; t++) {
            vb_start[t] = (uint32_t)n_verb;
            n_verb += tile_nv[t];
        }
        vb_start[sh.n_tiles] = (uint32_t)n_verb;
        auto is_verb = [&](int64_t t, int i, int c) {
            int bit = 4 * i + c / 64;
            return (vb_bits[t * 8 + bit / 32] >> (bit % 32)) & 1u;
        };
        auto sym = [&](int64_t t, int l, int k) -> int {
            int64_t rb = t / sh.n_cb, cb = t % sh.n_cb;
            int half = k >= 256;
            int c = k - 256 * half;
            int i = 2 * l + half;
            if (is_verb(t, i, c)) return 0;        // placeholder keeps lanes at 512 symbols
            return pidx[(w[(rb * 64 + i) * cols + cb * 256 + c] >> 7) & 255];
        };
        std::vector<uint64_t> hist(16, 0);
        {
            std::vector<std::vector<uint64_t>> ht(sh.n_rb);
            parallel_for(sh.n_rb, [&](int64_t rb) {
                std::vector<uint64_t> hh(16, 0);
                for (int64_t cb = 0; cb < sh.n_cb; cb++)
                    for (int l = 0; l < 32; l++)
                        for (int k = 0; k < 512; k++) hh[sym(rb * sh.n_cb + cb, l, k)]++;
                ht[rb] = hh;
            });
            for (int64_t rb = 0; rb < sh.n_rb; rb++)
                for (int s = 0; s < 16; s++) hist[s] += ht[rb][s];
        }
        uint8_t lens[16];
        uint16_t codes[16];
        lw_table tab;
        int n_sym = 0;
        if ((st = finish_table(16, hist, code, lens, codes, tab, n_sym))) return st;
        std::vector<uint32_t> tile_off;
        int32_t max_words = 0;
        encode_tiles(sh, 512, lens, codes, sym, tile_off, max_words, nullptr, nullptr);
        lw_image_header h = plan_image(LW_BF16_EXP, sh, tile_off[sh.n_tiles], n_verb, parts);
        h.n_sym = n_sym;
        h.max_words = max_words;
        h.n_pal = n_pal;
        h.code = code;
        std::unique_ptr<lw_bundle> b(new lw_bundle);
        uint64_t total = 0;
        for (int r = 0; r < LW_REG_COUNT; r++)
            if (h.bytes[r]) total = std::max<uint64_t>(total, lw_align_up(h.off[r] + h.bytes[r]));
        b->image.assign(total, 0);
        std::memcpy(region<uint32_t>(b->image, h, LW_REG_TILE_OFF), tile_off.data(), 4 * tile_off.size());
        *region<lw_table>(b->image, h, LW_REG_TABLE) = tab;
        std::memcpy(region<uint8_t>(b->image, h, LW_REG_PALETTE), palette, 16);
        fill_gputab(LW_BF16_EXP, tab, palette, h, region<lw_gputab>(b->image, h, LW_REG_GPUTAB));
        encode_tiles(sh, 512, lens, codes, sym, tile_off, max_words, &b->image, &h);
        std::memcpy(region<uint32_t>(b->image, h, LW_REG_VB_BITS), vb_bits.data(), 4 * vb_bits.size());
        std::memcpy(region<uint32_t>(b->image, h, LW_REG_VB_START), vb_start.data(), 4 * vb_start.size());
        uint32_t *sm = region<uint32_t>(b->image, h, LW_REG_SM);
        uint16_t *verb = n_verb ? region<uint16_t>(b->image, h, LW_REG_VERBATIM) : nullptr;
        parallel_for(sh.n_tiles, [&](int64_t t) {
            int64_t rb = t / sh.n_cb, cb = t % sh.n_cb;
            uint32_t *blk = sm + t * 4096;
            // sign+mantissa byte of tile row 2l+p, column 4g+b -> byte b of word (p*64+g)*32+l
            for (int p = 0; p < 2; p++)
                for (int l = 0; l < 32; l++) {
                    const uint16_t *row = w + (rb * 64 + 2 * l + p) * cols + cb * 256;
                    for (int g = 0; g < 64; g++) {
                        uint32_t v = 0;
                        for (int bb = 0; bb < 4; bb++) {
                            uint16_t x = row[4 * g + bb];
                            v |= (uint32_t)(((x >> 8) & 0x80) | (x & 0x7F)) << (8 * bb);
                        }
                        blk[(p * 64 + g) * 32 + l] = v;
                    }
                }
            uint32_t vo = vb_start[t];
            for (int i = 0; i < 64; i++)
                for (int s = 0; s < 4; s++)
                    if (is_verb(t, i, 64 * s)) {
                        std::memcpy(verb + (uint64_t)vo * 64, w + (rb * 64 + i) * cols + cb * 256 + 64 * s, 128);
                        vo++;
                    }
        });
        std::memcpy(b->image.data(), &h, sizeof(h));
        *out = b.release();
        return LW_OK;
    } catch (const std::bad_alloc &) {
        return lw_fail(LW_E_NOMEM, "host allocation failed");
    }
}

extern "C" lw_status lw_bundle_build_bf16(int64_t rows, int64_t cols, const uint16_t *w, lw_bundle **out)
{
    return build_bf16(rows, cols, w, LW_CODE_HUFFMAN, 0, out);
}

extern "C" lw_status lw_bundle_build_bf16_compact(int64_t rows, int64_t cols, const uint16_t *w, lw_bundle **out)
{
    return build_bf16(rows, cols, w, LW_CODE_COMPACT, 0, out);
}

extern "C" lw_status lw_bundle_build_bf16_opts(int64_t rows, int64_t cols, const uint16_t *w,
                                               const lw_build_opts *opts, lw_bundle **out)
{
    if (opts && opts->code == LW_CODE_LENS) {
        if (out) *out = nullptr;
        return lw_fail(LW_E_UNSUPPORTED, "bf16 bundles take the Huffman or compact code");
    }
    lw_status st = check_opts(opts, out);
    if (st) return st;
    return build_bf16(rows, cols, w, opts->code, opts->parts, out);
}

// ----------------------------------------------------------------- validate
const char *lw_region_name(int r)
{
    static const char *names[LW_REG_COUNT] = {"table", "gputab", "tile_off", "words", "dm", "palette",
                                             "sm", "vb_bits", "vb_start", "verbatim", "split", "work"};
    return r >= 0 && r < LW_REG_COUNT ? names[r] : "?";
}

uint32_t lw_regions_needed(const lw_image_header &h, int op)
{
    const bool bf16 = h.kind == LW_BF16_EXP;
    uint32_t m = 1u << LW_REG_GPUTAB | 1u << LW_REG_TILE_OFF | 1u << LW_REG_WORDS | 1u << LW_REG_SPLIT;
    if (op == LW_OP_ANY) m |= 1u << LW_REG_TABLE;
    if (bf16) {
        m |= 1u << LW_REG_SM | 1u << LW_REG_VB_BITS | 1u << LW_REG_VB_START;
        if (op == LW_OP_ANY) m |= 1u << LW_REG_PALETTE;
        if (h.n_verbatim > 0) m |= 1u << LW_REG_VERBATIM;
    } else if (op != LW_OP_DECODE) {
        m |= 1u << LW_REG_DM;                     // scales of the dequantisation
    }
    if (op != LW_OP_DECODE && h.work_groups > 1) m |= 1u << LW_REG_WORK;   // split-column reduction
    return m;
}

static lw_status validate_image(const uint8_t *img, size_t bytes)
{
    if (bytes < LW_HEADER_BYTES) return lw_fail(LW_E_FORMAT, "image shorter than its header");
    lw_image_header h;
    std::memcpy(&h, img, sizeof(h));
    if (h.magic != LW_MAGIC || h.version != LW_VERSION) return lw_fail(LW_E_FORMAT, "bad magic/version");
    if (h.kind < LW_Q4_PAIR || h.kind > LW_BF16_EXP) return lw_fail(LW_E_FORMAT, "bad kind");
    if (h.rows <= 0 || h.cols <= 0 || h.rows % 64 || h.cols % 256) return lw_fail(LW_E_FORMAT, "bad shape");
    if (h.n_rb != h.rows / 64 || h.n_cb != h.cols / 256 || h.n_tiles != (int64_t)h.n_rb * h.n_cb)
        return lw_fail(LW_E_FORMAT, "inconsistent tile counts");
    if (h.spl != (h.kind == LW_Q4_PAIR ? 256 : 512)) return lw_fail(LW_E_FORMAT, "bad symbols per lane");
    if (h.code < LW_CODE_HUFFMAN || h.code > LW_CODE_LENS) return lw_fail(LW_E_FORMAT, "unknown code kind");
    uint64_t prev_end = LW_HEADER_BYTES;
    for (int r = 0; r < LW_REG_COUNT; r++) {
        if (!h.bytes[r]) continue;
        if (h.off[r] % LW_ALIGN || h.off[r] < prev_end || h.off[r] + h.bytes[r] > bytes)
            return lw_fail(LW_E_FORMAT, "region out of bounds: " + std::to_string(r));
        prev_end = h.off[r] + h.bytes[r];
    }
    const uint32_t need = lw_regions_needed(h, LW_OP_ANY);
    for (int r = 0; r < LW_REG_COUNT; r++)
        if ((need >> r & 1u) && !h.bytes[r]) return lw_fail(LW_E_FORMAT, std::string("missing region ") + lw_region_name(r));
    if (h.bytes[LW_REG_TABLE] != sizeof(lw_table) || h.bytes[LW_REG_GPUTAB] != sizeof(lw_gputab))
        return lw_fail(LW_E_FORMAT, "table region size");
    if (h.bytes[LW_REG_TILE_OFF] != 4u * (uint64_t)(h.n_tiles + 1)) return lw_fail(LW_E_FORMAT, "tile_off size");
    if (h.parts != 1 && h.parts != 2 && h.parts != 4 && h.parts != 8) return lw_fail(LW_E_FORMAT, "bad parts per row");
    if (h.bytes[LW_REG_SPLIT] != 2u * LW_LANES * (uint64_t)h.n_tiles * (uint64_t)(2 * h.parts - 1))
        return lw_fail(LW_E_FORMAT, "split size");
    if (h.kind != LW_BF16_EXP && h.bytes[LW_REG_DM] != 256u * (uint64_t)h.n_tiles)
        return lw_fail(LW_E_FORMAT, "dm size");
    if (h.kind == LW_BF16_EXP &&
        (h.bytes[LW_REG_SM] != 16384u * (uint64_t)h.n_tiles || h.bytes[LW_REG_VB_BITS] != 32u * (uint64_t)h.n_tiles ||
         h.bytes[LW_REG_VB_START] != 4u * (uint64_t)(h.n_tiles + 1) || h.bytes[LW_REG_VERBATIM] != 128u * (uint64_t)h.n_verbatim))
        return lw_fail(LW_E_FORMAT, "bf16 region sizes");
    // table: lengths <= 11, Kraft sum, consistent canonical arrays
    lw_table t;
    std::memcpy(&t, img + h.off[LW_REG_TABLE], sizeof(t));
    int n_alpha = h.kind == LW_Q4_PAIR ? 256 : (h.kind == LW_Q6_SINGLE ? 64 : 16);
    uint64_t kraft = 0;
    int nsym = 0, lmin = 0, lmax = 0;
    uint32_t code = 0;
    for (int L = 1; L <= LW_MAXLEN; L++) {
        code = (code + (L > 1 ? t.count[L - 1] : 0)) << 1;
        if (t.first[L] != code) return lw_fail(LW_E_TABLE, "first[] not canonical");
        if (t.offset[L] != nsym) return lw_fail(LW_E_TABLE, "offset[] inconsistent");
        if (t.limit[L] != (uint16_t)(((uint32_t)t.first[L] + t.count[L]) << (LW_MAXLEN - L)))
            return lw_fail(LW_E_TABLE, "limit[] inconsistent");
        kraft += (uint64_t)t.count[L] << (LW_MAXLEN - L);
        nsym += t.count[L];
        if (t.count[L]) {
            if (!lmin) lmin = L;
            lmax = L;
        }
    }
    if (t.count[0]) return lw_fail(LW_E_TABLE, "count[0] nonzero");
    if (nsym < 1 || nsym > n_alpha) return lw_fail(LW_E_TABLE, "symbol count");
    if (kraft > 2048) return lw_fail(LW_E_TABLE, "Kraft sum violated");
    if (nsym != h.n_sym || lmin != h.min_len || lmax != h.max_len) return lw_fail(LW_E_TABLE, "header/table mismatch");
    for (int i = 0; i < nsym; i++)
        if (t.sym_sorted[i] >= n_alpha) return lw_fail(LW_E_TABLE, "symbol out of alphabet");
    const lw_gputab *g = reinterpret_cast<const lw_gputab *>(img + h.off[LW_REG_GPUTAB]);
    for (int r = 0; r <= lmax - lmin; r++) {
        int L = lmin + r;
        if ((int)g->len[r] != L || g->base[r] != (int32_t)t.offset[L] - (int32_t)t.first[L])
            return lw_fail(LW_E_FORMAT, "gpu table mismatch");
    }
    for (int L = lmin; L < lmax; L++)
        if (g->limlj[L - lmin] != ((uint32_t)t.limit[L] << 21)) return lw_fail(LW_E_FORMAT, "gpu limits mismatch");
    {
        lw_plan want;
        lw_make_plan(t, lmin, lmax, want);
        if (std::memcmp(&want, &g->plan, sizeof(want)) != 0) return lw_fail(LW_E_FORMAT, "comparison plan mismatch");
    }
    // tile offsets: start at 0, grow by whole word rows, end at the word count
    const uint32_t *to = reinterpret_cast<const uint32_t *>(img + h.off[LW_REG_TILE_OFF]);
    if (to[0] != 0) return lw_fail(LW_E_FORMAT, "tile_off[0] != 0");
    int32_t wmax = 0;
    for (int64_t i = 0; i < h.n_tiles; i++) {
        if (to[i + 1] < to[i] || (to[i + 1] - to[i]) % 32) return lw_fail(LW_E_FORMAT, "tile_off not monotone rows");
        wmax = std::max<int32_t>(wmax, (int32_t)((to[i + 1] - to[i]) / 32));
    }
    if ((uint64_t)to[h.n_tiles] * 4u != h.bytes[LW_REG_WORDS]) return lw_fail(LW_E_FORMAT, "words size");
    // each part of a lane stream starts inside the stream, 1 to 11 bits per
    // symbol after the start of the part before it
    const uint16_t *sp = reinterpret_cast<const uint16_t *>(img + h.off[LW_REG_SPLIT]);
    const int nparts = 2 * h.parts;
    const uint32_t per = (uint32_t)(h.spl / nparts);
    for (int64_t i = 0; i < h.n_tiles; i++) {
        const uint32_t lane_words = (to[i + 1] - to[i]) / 32u;
        for (int l = 0; l < LW_LANES; l++) {
            uint32_t prev = 0;
            for (int k = 1; k < nparts; k++) {
                const uint32_t v = sp[(i * (nparts - 1) + k - 1) * LW_LANES + l];
                if (v < prev + per || v > prev + per * LW_MAXLEN || v > 32u * lane_words)
                    return lw_fail(LW_E_FORMAT, "part start outside the lane stream");
                prev = v;
            }
        }
    }
    if (wmax != h.max_words) return lw_fail(LW_E_FORMAT, "max_words mismatch");
    // a lane can hold at most symbols_per_lane codes of 11 bits
    if ((int64_t)wmax * 32 > (int64_t)h.spl * LW_MAXLEN + 31) return lw_fail(LW_E_FORMAT, "tile longer than possible");
    if (h.kind == LW_BF16_EXP) {
        const uint32_t *vs = reinterpret_cast<const uint32_t *>(img + h.off[LW_REG_VB_START]);
        const uint32_t *vb = reinterpret_cast<const uint32_t *>(img + h.off[LW_REG_VB_BITS]);
        if (vs[0] != 0) return lw_fail(LW_E_FORMAT, "vb_start[0] != 0");
        for (int64_t i = 0; i < h.n_tiles; i++) {
            uint32_t pc = 0;
            for (int j = 0; j < 8; j++) pc += (uint32_t)__builtin_popcount(vb[i * 8 + j]);
            if (vs[i + 1] != vs[i] + pc) return lw_fail(LW_E_FORMAT, "vb_start inconsistent");
        }
        if ((int64_t)vs[h.n_tiles] != h.n_verbatim) return lw_fail(LW_E_FORMAT, "verbatim count");
        if (h.n_pal < 1 || h.n_pal > 16 || nsym > h.n_pal) return lw_fail(LW_E_FORMAT, "palette size");
    }
    const int32_t groups = lw_work_groups(h.n_cb, h.parts);
    if (h.work_groups != groups) return lw_fail(LW_E_FORMAT, "workspace groups");
    if (h.bytes[LW_REG_WORK] < lw_work_bytes(groups, h.rows))
        return lw_fail(LW_E_FORMAT, "workspace too small");
    return LW_OK;
}

extern "C" lw_status lw_bundle_validate(const lw_bundle *b)
{
    if (!b) return lw_fail(LW_E_ARG, "bundle is null");
    return validate_image(b->image.data(), b->image.size());
}

extern "C" lw_status lw_bundle_load(const void *image, size_t bytes, lw_bundle **out)
{
    if (!out) return lw_fail(LW_E_ARG, "out is null");
    *out = nullptr;
    if (!image) return lw_fail(LW_E_ARG, "image is null");
    lw_status st = validate_image(static_cast<const uint8_t *>(image), bytes);
    if (st) return st;
    try {
        std::unique_ptr<lw_bundle> b(new lw_bundle);
        b->image.assign(static_cast<const uint8_t *>(image), static_cast<const uint8_t *>(image) + bytes);
        // the workspace must start zeroed
        lw_image_header h;
        std::memcpy(&h, b->image.data(), sizeof(h));
        if (h.bytes[LW_REG_WORK]) std::memset(b->image.data() + h.off[LW_REG_WORK], 0, h.bytes[LW_REG_WORK]);
        *out = b.release();
        return LW_OK;
    } catch (const std::bad_alloc &) {
        return lw_fail(LW_E_NOMEM, "host allocation failed");
    }
}

extern "C" lw_status lw_bundle_get_info(const lw_bundle *b, lw_bundle_info *info)
{
    if (!b || !info) return lw_fail(LW_E_ARG, "null argument");
    lw_image_header h;
    std::memcpy(&h, b->image.data(), sizeof(h));
    std::memset(info, 0, sizeof(*info));
    info->kind = h.kind;
    info->bits = h.bits;
    info->rows = h.rows;
    info->cols = h.cols;
    info->n_tiles = h.n_tiles;
    info->n_rb = h.n_rb;
    info->n_cb = h.n_cb;
    info->symbols_per_lane = h.spl;
    info->n_symbols = h.n_sym;
    info->min_len = h.min_len;
    info->max_len = h.max_len;
    info->max_words = h.max_words;
    info->parts = h.parts;
    info->n_palette = h.n_pal;
    info->n_verbatim = h.n_verbatim;
    const lw_table *t = reinterpret_cast<const lw_table *>(b->image.data() + h.off[LW_REG_TABLE]);
    for (int L = 0; L < 12; L++) info->count_per_len[L] = t->count[L];
    for (int r = 0; r < LW_REG_COUNT; r++) {
        info->region_offset[r] = h.off[r];
        info->region_bytes[r] = h.bytes[r];
    }
    info->image_bytes = b->image.size();
    info->coded_bytes = h.coded_bytes;
    info->twin_bytes = h.twin_bytes;
    info->code = h.code;
    return LW_OK;
}

extern "C" lw_status lw_bundle_image(const lw_bundle *b, const void **image, size_t *bytes)
{
    if (!b || !image || !bytes) return lw_fail(LW_E_ARG, "null argument");
    *image = b->image.data();
    *bytes = b->image.size();
    return LW_OK;
}

extern "C" lw_status lw_bundle_region(const lw_bundle *b, int r, const void **ptr, size_t *bytes)
{
    if (!b || !ptr || !bytes) return lw_fail(LW_E_ARG, "null argument");
    if (r < 0 || r >= LW_REG_COUNT) return lw_fail(LW_E_ARG, "no such region");
    lw_image_header h;
    std::memcpy(&h, b->image.data(), sizeof(h));
    *ptr = h.bytes[r] ? b->image.data() + h.off[r] : nullptr;
    *bytes = h.bytes[r];
    return LW_OK;
}

extern "C" void lw_bundle_free(lw_bundle *b) { delete b; }

extern "C" lw_status lw_twin_build(const uint8_t *codes, int bits, int64_t rows, int64_t cols,
                                   const uint16_t *d, const uint16_t *m, uint8_t *twin, uint32_t *dm)
{
    if (!codes || !d || !m || !twin || !dm) return lw_fail(LW_E_ARG, "null argument");
    if (bits != 4) return lw_fail(LW_E_ARG, "twin supports 4-bit codes");
    if (rows <= 0 || cols <= 0 || cols % 256) return lw_fail(LW_E_SHAPE, "cols must be a multiple of 256");
    std::atomic<int> bad(0);
    parallel_for(rows, [&](int64_t r) {
        const uint8_t *q = codes + r * cols;
        uint8_t *o = twin + r * (cols / 2);
        for (int64_t c = 0; c < cols; c += 2) {
            if ((q[c] | q[c + 1]) > 15) bad = 1;
            o[c / 2] = (uint8_t)((q[c] & 15) | (q[c + 1] << 4));
        }
        for (int64_t s = 0; s < cols / 256; s++)
            dm[r * (cols / 256) + s] = (uint32_t)d[r * (cols / 256) + s] | ((uint32_t)m[r * (cols / 256) + s] << 16);
    });
    if (bad) return lw_fail(LW_E_ARG, "code >= 16");
    return LW_OK;
}

/* Tile-transposed fixed-width packing ("Software-Defined Bandwidth
 * Expansion", IV-A storage and IV-B layout): 32/bits codes per 32-bit word,
 * the code of the lowest column in the lowest bits; word (t, j, r) holds
 * columns [j*32/bits, (j+1)*32/bits) of row 64t + r and sits at index
 * (t*WPR + j)*64 + r, WPR = cols*bits/32; scales at (t*(cols/256) + g)*64 + r. */
extern "C" lw_status lw_skip_pack(const uint8_t *codes, int bits, int64_t rows, int64_t cols,
                                  const uint16_t *d, const uint16_t *m, uint32_t *words, uint32_t *dm)
{
    if (!codes || !d || !m || !words || !dm) return lw_fail(LW_E_ARG, "null argument");
    if (bits != 2 && bits != 4 && bits != 8) return lw_fail(LW_E_ARG, "bits must be 2, 4 or 8");
    if (rows <= 0 || cols <= 0 || rows % 64 || cols % 256)
        return lw_fail(LW_E_SHAPE, "rows must be a multiple of 64 and cols of 256");
    const int per = 32 / bits;
    const int64_t wpr = cols / per, ng = cols / 256;
    const unsigned top = (1u << bits) - 1u;
    std::atomic<int> bad(0);
    parallel_for(rows, [&](int64_t r) {
        const uint8_t *q = codes + r * cols;
        const int64_t t = r >> 6, rr = r & 63;
        uint32_t *wt = words + t * wpr * 64 + rr;
        for (int64_t j = 0; j < wpr; j++) {
            uint32_t w = 0;
            for (int i = per - 1; i >= 0; i--) {
                const uint8_t c = q[j * per + i];
                if (c > top) bad = 1;
                w = (w << bits) | (c & top);
            }
            wt[j * 64] = w;
        }
        uint32_t *dt = dm + t * ng * 64 + rr;
        for (int64_t g = 0; g < ng; g++) dt[g * 64] = (uint32_t)d[r * ng + g] | ((uint32_t)m[r * ng + g] << 16);
    });
    if (bad) return lw_fail(LW_E_ARG, "code does not fit in the bit width");
    return LW_OK;
}

/* ------------------------------------------------------------------ rANS twin
 * The rANS lane coder of the decode-cost ablation ("LazyWeights", section
 * "Decoder hardware": Huffman against rANS).  Format: frequencies scaled to
 * 2^11 (absent symbols 0, present ones at least 1, each its rounded share,
 * then the largest entries nudged by one until the sum is exact), one stream
 * per tile row (or two, one per half of the row's columns: stream h*64 + r)
 * with 32-bit state in [2^16, 2^32) and 16-bit renormalisation, a tile block
 * = ns head states then the chunks in 16-bit units, chunk k of stream s at
 * unit ns*k + s, zero-padded to an even per-tile chunk count. */
namespace {

constexpr uint32_t RANS_PB = 11, RANS_M = 1u << RANS_PB, RANS_L = 1u << 16;

bool rans_quantise(const std::vector<uint64_t> &hist, std::vector<uint32_t> &f)
{
    const size_t n = hist.size();
    uint64_t total = 0;
    for (uint64_t c : hist) total += c;
    f.assign(n, 0);
    if (!total) return false;
    int64_t sum = 0;
    for (size_t s = 0; s < n; s++) {
        if (!hist[s]) continue;
        // round(hist * M / total), halves up, never below 1
        const uint64_t num = hist[s] * RANS_M, q = num / total, rem = num % total;
        f[s] = std::max<uint64_t>(1, q + (2 * rem >= total ? 1 : 0));
        sum += f[s];
    }
    while (sum != (int64_t)RANS_M) {
        const bool over = sum > (int64_t)RANS_M;
        size_t best = n;
        for (size_t s = 0; s < n; s++) {
            const uint32_t v = f[s];
            if (v == 0 || (over && v == 1)) continue;
            if (best == n || v > f[best]) best = s;                 // strict: the smaller symbol keeps a tie
        }
        if (best == n) return false;
        if (over) { f[best]--; sum--; }
        else { f[best]++; sum++; }
    }
    return true;
}

// Encode one stream; chunks come out in emission order and are reversed
// by the caller's placement.  Returns the chunk count.
int rans_encode_row(const uint16_t *sym, int n, const uint32_t *f, const uint32_t *cum, uint32_t &state,
                    uint16_t *chunks)
{
    uint32_t x = RANS_L;
    int k = 0;
    for (int i = n - 1; i >= 0; i--) {
        const uint32_t fs = f[sym[i]];
        const uint64_t bound = (uint64_t)fs << (32 - RANS_PB);    // 2^21 f: the coded state stays < 2^32
        while (x >= bound) {
            chunks[k++] = (uint16_t)x;
            x >>= 16;
        }
        const uint32_t q = x / fs;
        x = (q << RANS_PB) + (x - q * fs) + cum[sym[i]];
    }
    state = x;
    return k;
}

}  // namespace

extern "C" lw_status lw_rans_build(int kind, int64_t rows, int64_t cols, const uint8_t *codes, int halves,
                                   uint16_t *freq, uint32_t *lut, uint32_t *tile_off, uint32_t *words,
                                   int64_t words_cap, int64_t *n_words, int32_t *max_tile_words)
{
    if (!codes || !freq || !lut || !tile_off || !n_words || !max_tile_words) return lw_fail(LW_E_ARG, "null argument");
    if (kind != LW_Q4_PAIR && kind != LW_Q6_SINGLE) return lw_fail(LW_E_ARG, "kind must be LW_Q4_PAIR or LW_Q6_SINGLE");
    if (halves != 1 && halves != 2) return lw_fail(LW_E_ARG, "halves must be 1 or 2");
    if (rows <= 0 || cols <= 0 || rows % 64 || cols % 256)
        return lw_fail(LW_E_SHAPE, "rows must be a multiple of 64 and cols of 256");
    const bool q4 = kind == LW_Q4_PAIR;
    const int spr = q4 ? 128 : 256, n_alpha = q4 ? 256 : 64;
    const int ns = 64 * halves, sps = spr / halves;          // streams a tile, symbols a stream
    // stream s = h*64 + r of tile t: half h of row r's symbols
    auto stream = [&](const std::vector<uint16_t> &sy, int64_t t, int st) {
        return sy.data() + (t * 64 + (st & 63)) * spr + (st >> 6) * sps;
    };
    const int64_t ncb = cols / 256, nt = (rows / 64) * ncb;
    if (nt > 0x7FFFFFFF) return lw_fail(LW_E_SHAPE, "too many tiles");
    const unsigned top = q4 ? 15u : 63u;

    // symbols: stream (t, r) = row r of tile t, pairs of columns (2i, 2i+1) or single codes
    std::vector<uint16_t> syms;
    try { syms.resize((size_t)nt * 64 * spr); } catch (...) { return lw_fail(LW_E_NOMEM, "symbol buffer"); }
    std::atomic<int> bad(0);
    parallel_for(rows, [&](int64_t r) {
        const uint8_t *q = codes + r * cols;
        for (int64_t cb = 0; cb < ncb; cb++) {
            uint16_t *o = syms.data() + (((r >> 6) * ncb + cb) * 64 + (r & 63)) * spr;
            const uint8_t *c = q + cb * 256;
            for (int i = 0; i < spr; i++) {
                const unsigned lo = q4 ? c[2 * i] : c[i], hi = q4 ? c[2 * i + 1] : 0u;
                if (lo > top || hi > top) bad = 1;
                o[i] = (uint16_t)(q4 ? (lo | hi << 4) : lo);
            }
        }
    });
    if (bad) return lw_fail(LW_E_ARG, "code out of range");

    std::vector<uint64_t> hist(n_alpha, 0);
    for (uint16_t s : syms) hist[s]++;
    std::vector<uint32_t> f;
    if (!rans_quantise(hist, f)) return lw_fail(LW_E_TABLE, "frequencies cannot be scaled to 2^11");
    std::vector<uint32_t> cum(n_alpha + 1, 0);
    for (int s = 0; s < n_alpha; s++) cum[s + 1] = cum[s] + f[s];
    for (int s = 0; s < n_alpha; s++) freq[s] = (uint16_t)f[s];
    for (int s = 0; s < n_alpha; s++)
        for (uint32_t slot = cum[s]; slot < cum[s + 1]; slot++) {
            lut[2 * slot] = f[s] | (uint32_t)s << 24;
            lut[2 * slot + 1] = slot - cum[s];
        }

    // pass 1: chunk count of every tile (even), then offsets
    std::vector<int32_t> kt((size_t)nt);
    parallel_for(nt, [&](int64_t t) {
        std::vector<uint16_t> ch(sps);
        int kmax = 0;
        for (int r = 0; r < ns; r++) {
            uint32_t st;
            kmax = std::max(kmax, rans_encode_row(stream(syms, t, r), sps, f.data(), cum.data(), st, ch.data()));
        }
        kt[t] = kmax + (kmax & 1);
    });
    int64_t pos = 0;
    int32_t tmax = 0;
    for (int64_t t = 0; t < nt; t++) {
        if (pos > 0xFFFFFFFFll) return lw_fail(LW_E_SHAPE, "word offsets exceed 32 bits");
        tile_off[t] = (uint32_t)pos;
        pos += ns + (int64_t)ns / 2 * kt[t];
        tmax = std::max<int32_t>(tmax, ns + ns / 2 * kt[t]);
    }
    if (pos > 0xFFFFFFFFll) return lw_fail(LW_E_SHAPE, "word offsets exceed 32 bits");
    tile_off[nt] = (uint32_t)pos;
    *n_words = pos;
    *max_tile_words = tmax;
    if (!words) return LW_OK;
    if (words_cap < pos) return lw_fail(LW_E_ARG, "words buffer too small");

    // pass 2: the blocks
    parallel_for(nt, [&](int64_t t) {
        std::vector<uint16_t> ch(sps);
        uint32_t *blk = words + tile_off[t];
        std::memset(blk, 0, sizeof(uint32_t) * (size_t)(ns + (int64_t)ns / 2 * kt[t]));
        uint16_t *area = reinterpret_cast<uint16_t *>(blk + ns);   // little-endian 16-bit view
        for (int r = 0; r < ns; r++) {
            uint32_t st;
            const int k = rans_encode_row(stream(syms, t, r), sps, f.data(), cum.data(), st, ch.data());
            blk[r] = st;
            for (int j = 0; j < k; j++) area[(size_t)ns * j + r] = ch[k - 1 - j];   // the decoder reads the last emitted first
        }
    });
    return LW_OK;
}
