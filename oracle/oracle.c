/*
 * oracle.c -- plain, slow CPU reference of lane-interleaved, length-limited
 * canonical Huffman coding of LLM weight codes and of the GEMV over them.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the product library (decode_gemv_amd/csrc),
 * and the product never calls it.
 *
 * Everything is single-threaded, scalar C with no blocking or reordering
 * beyond what the method defines.  Sources, cited by page title and place:
 *
 *   [LW]  "LazyWeights: Decode-on-Demand Edge LLMs" -- section "2 . Code them",
 *         section "3 . Decode on demand", Fig. 3 (bundle layout, decode unit).
 *   [UW]  "Unweight: Compressing LLM Weights for Faster Inference" -- sections
 *         "Understanding BF16 weight structure" and "The exponent's exploitable
 *         redundancy" (exponent palette, 64-weight verbatim rows).
 *   [SDB] "Software-Defined Bandwidth Expansion ..." -- sections IV-A/IV-C
 *         (grouped storage w = d*q - m, dense dequantise-then-multiply check;
 *         IV-B tile-transposed layout and IV-C tile skipping and its ledger).
 *
 * Readings of points the pages leave open are stated at each function.
 *
 * Parity pins: every function here is pinned by the CPU tests (Kraft
 * equality, brute-force optimal lengths, dyadic closed form, textbook heap
 * Huffman when the limit does not bind, round trip on every tile, bit-by-bit
 * decoding, naive dense matvec, closed-form special cases).  No function is
 * left unpinned.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define OR_MAXLEN 11          /* [LW] section 2: no code is longer than 11 bits     */
#define OR_TILE_ROWS 64       /* [LW] section 2: tiles of 64 rows by 256 columns,   */
                              /* each lane holding two of the rows                 */
#define OR_TILE_COLS 256
#define OR_LANES 32

enum { OR_Q4 = 1, OR_Q6 = 2, OR_BF16 = 3 };

/* ------------------------------------------------------------------ */
/* Symbols.                                                             */
/* ------------------------------------------------------------------ */

/* Symbols one lane carries: two rows of 256 codes.  4-bit codes are coded
 * in pairs (two adjacent 4-bit codes form one symbol, [LW] section 2), so
 * 256 pair symbols;
 * 6-bit codes and bf16 exponent indices are coded singly, so 512. */
int or_symbols_per_lane(int kind) { return kind == OR_Q4 ? 256 : 512; }

int or_alphabet(int kind) { return kind == OR_Q4 ? 256 : (kind == OR_Q6 ? 64 : 16); }

/* Reading: lane l of tile (rb, cb) carries rows 64*rb + 2l and 64*rb + 2l + 1,
 * row 2l first, each in column order.  A pair symbol is the codes of columns
 * 2k (low nibble) and 2k+1 (high nibble) of one row.  Tiles are numbered
 * row-band-major, t = rb * (cols/256) + cb.
 * syms has n_tiles * 32 * spl entries, laid out [t][lane][k]. */
void or_symbolise_q(int kind, int64_t rows, int64_t cols, const uint8_t *q, uint16_t *syms)
{
    int64_t nrb = rows / OR_TILE_ROWS, ncb = cols / OR_TILE_COLS;
    int spl = or_symbols_per_lane(kind);
    for (int64_t rb = 0; rb < nrb; rb++)
        for (int64_t cb = 0; cb < ncb; cb++) {
            int64_t t = rb * ncb + cb;
            for (int l = 0; l < OR_LANES; l++) {
                uint16_t *out = syms + (t * OR_LANES + l) * spl;
                int k = 0;
                for (int half = 0; half < 2; half++) {
                    int64_t r = rb * OR_TILE_ROWS + 2 * l + half;
                    const uint8_t *row = q + r * cols + cb * OR_TILE_COLS;
                    if (kind == OR_Q4) {
                        for (int c = 0; c < OR_TILE_COLS; c += 2)
                            out[k++] = (uint16_t)(row[c] | (row[c + 1] << 4));
                    } else {
                        for (int c = 0; c < OR_TILE_COLS; c++)
                            out[k++] = row[c];
                    }
                }
            }
        }
}

/* Inverse of or_symbolise_q. */
void or_unsymbolise_q(int kind, int64_t rows, int64_t cols, const uint16_t *syms, uint8_t *q)
{
    int64_t nrb = rows / OR_TILE_ROWS, ncb = cols / OR_TILE_COLS;
    int spl = or_symbols_per_lane(kind);
    for (int64_t rb = 0; rb < nrb; rb++)
        for (int64_t cb = 0; cb < ncb; cb++) {
            int64_t t = rb * ncb + cb;
            for (int l = 0; l < OR_LANES; l++) {
                const uint16_t *in = syms + (t * OR_LANES + l) * spl;
                int k = 0;
                for (int half = 0; half < 2; half++) {
                    int64_t r = rb * OR_TILE_ROWS + 2 * l + half;
                    uint8_t *row = q + r * cols + cb * OR_TILE_COLS;
                    if (kind == OR_Q4) {
                        for (int c = 0; c < OR_TILE_COLS; c += 2) {
                            row[c] = (uint8_t)(in[k] & 15);
                            row[c + 1] = (uint8_t)(in[k] >> 4);
                            k++;
                        }
                    } else {
                        for (int c = 0; c < OR_TILE_COLS; c++)
                            row[c] = (uint8_t)in[k++];
                    }
                }
            }
        }
}

/* One code table serves a whole matrix ([LW] section 2), so the histogram
 * is taken over all symbols of the matrix. */
void or_histogram(const uint16_t *syms, int64_t n, int n_alpha, uint64_t *counts)
{
    for (int s = 0; s < n_alpha; s++) counts[s] = 0;
    for (int64_t i = 0; i < n; i++) counts[syms[i]]++;
}

/* ------------------------------------------------------------------ */
/* Code lengths: package-merge (Larmore & Hirschberg), limit L.          */
/* ------------------------------------------------------------------ */
/* Reading: the pages fix only the 11-bit limit.  The lengths are the optimal
 * length-limited prefix code found by package-merge.  Ties are broken as
 * follows so that the result is reproducible:
 *   - leaves are sorted by (count ascending, symbol ascending);
 *   - a level's packages pair adjacent items (0,1), (2,3), ... of the
 *     previous list, an odd last item being dropped;
 *   - leaves and packages merge by weight, a leaf first on equal weights;
 *   - the first 2n-2 items of the last list are selected, and a symbol's
 *     length is the number of selected items that contain it.
 * A matrix with a single used symbol gets length 1.
 * Each item carries, explicitly, how many times each symbol occurs in it. */
typedef struct {
    uint64_t w;
    uint16_t *mult;           /* n_alpha multiplicities */
} or_item;

typedef struct { uint64_t c; int s; } or_leaf;

static int leaf_less(const or_leaf *a, const or_leaf *b)
{
    if (a->c != b->c) return a->c < b->c;
    return a->s < b->s;
}

/* returns 0 on success, -1 if the alphabet cannot be coded within L bits */
int or_package_merge(int n_alpha, const uint64_t *counts, int L, uint8_t *lens)
{
    int n = 0;
    or_leaf *leaves = (or_leaf *)malloc(sizeof(or_leaf) * (size_t)(n_alpha > 0 ? n_alpha : 1));
    for (int s = 0; s < n_alpha; s++) {
        lens[s] = 0;
        if (counts[s] > 0) { leaves[n].c = counts[s]; leaves[n].s = s; n++; }
    }
    if (n == 0) { free(leaves); return 0; }
    if (n == 1) { lens[leaves[0].s] = 1; free(leaves); return 0; }
    if (L < 31 && ((int64_t)1 << L) < n) { free(leaves); return -1; }
    /* insertion sort, (count, symbol) ascending */
    for (int i = 1; i < n; i++) {
        or_leaf v = leaves[i];
        int j = i - 1;
        while (j >= 0 && leaf_less(&v, &leaves[j])) { leaves[j + 1] = leaves[j]; j--; }
        leaves[j + 1] = v;
    }
    int cap = 2 * n + 2;
    or_item *list = (or_item *)calloc((size_t)cap, sizeof(or_item));
    or_item *next = (or_item *)calloc((size_t)cap, sizeof(or_item));
    for (int i = 0; i < cap; i++) {
        list[i].mult = (uint16_t *)calloc((size_t)n_alpha, sizeof(uint16_t));
        next[i].mult = (uint16_t *)calloc((size_t)n_alpha, sizeof(uint16_t));
    }
    int len_list = n;
    for (int i = 0; i < n; i++) {
        list[i].w = leaves[i].c;
        memset(list[i].mult, 0, sizeof(uint16_t) * (size_t)n_alpha);
        list[i].mult[leaves[i].s] = 1;
    }
    for (int level = 1; level < L; level++) {
        /* packages of adjacent pairs of the current list */
        int npk = len_list / 2;
        or_item *pk = (or_item *)calloc((size_t)(npk > 0 ? npk : 1), sizeof(or_item));
        for (int p = 0; p < npk; p++) {
            pk[p].w = list[2 * p].w + list[2 * p + 1].w;
            pk[p].mult = (uint16_t *)calloc((size_t)n_alpha, sizeof(uint16_t));
            for (int s = 0; s < n_alpha; s++)
                pk[p].mult[s] = (uint16_t)(list[2 * p].mult[s] + list[2 * p + 1].mult[s]);
        }
        /* merge leaves and packages by weight, leaf first on ties */
        int i = 0, p = 0, o = 0;
        while (i < n || p < npk) {
            int take_leaf;
            if (i >= n) take_leaf = 0;
            else if (p >= npk) take_leaf = 1;
            else take_leaf = leaves[i].c <= pk[p].w;
            if (take_leaf) {
                next[o].w = leaves[i].c;
                memset(next[o].mult, 0, sizeof(uint16_t) * (size_t)n_alpha);
                next[o].mult[leaves[i].s] = 1;
                i++;
            } else {
                next[o].w = pk[p].w;
                memcpy(next[o].mult, pk[p].mult, sizeof(uint16_t) * (size_t)n_alpha);
                p++;
            }
            o++;
        }
        for (int q = 0; q < npk; q++) free(pk[q].mult);
        free(pk);
        or_item *tmp = list; list = next; next = tmp;
        len_list = o;
    }
    int take = 2 * n - 2;
    int lens_acc[1024];
    for (int s = 0; s < n_alpha; s++) lens_acc[s] = 0;
    for (int k = 0; k < take && k < len_list; k++)
        for (int s = 0; s < n_alpha; s++) lens_acc[s] += list[k].mult[s];
    for (int s = 0; s < n_alpha; s++) lens[s] = (uint8_t)lens_acc[s];
    for (int i2 = 0; i2 < cap; i2++) { free(list[i2].mult); free(next[i2].mult); }
    free(list); free(next); free(leaves);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Code lengths of the opt-in compact code.                              */
/* ------------------------------------------------------------------ */
/* The bundles' default lengths are package-merge's above.  The compact code
 * is an option of the product (a smaller decoder comparison plan at a small
 * cost in bits); the oracle builds it so the option can be checked too.  It
 * is the cheapest prefix code (least
 * total bits sum count * length) among those with lengths <= 11 and at most
 * four distinct lengths, of which the three shorter are <= 8 (so a decoder
 * needs three comparisons of the top 8 peek bits).  Search and ties:
 *   - rank the used symbols by (count descending, symbol ascending);
 *   - for every length set a < b < c <= 8, c < d <= 11, in ascending
 *     lexicographic order, and every split of the ranks into n1 at length
 *     a, n2 at b (n1, n2 ascending), give length c to as many of the
 *     remaining ranks as the Kraft sum (<= 1) allows and d to the rest;
 *   - keep the first split whose total is strictly below every earlier one.
 * Giving c to more ranks never costs bits, so the search is exhaustive over
 * the allowed codes.  A single used symbol gets length 1.  Returns 0, or -1
 * if more than 256 symbols are used (no such code exists). */
int or_compact_lengths(int n_alpha, const uint64_t *counts, uint8_t *lens)
{
    int n = 0;
    or_leaf *rank = (or_leaf *)malloc(sizeof(or_leaf) * (size_t)(n_alpha > 0 ? n_alpha : 1));
    for (int s = 0; s < n_alpha; s++) {
        lens[s] = 0;
        if (counts[s] > 0) { rank[n].c = counts[s]; rank[n].s = s; n++; }
    }
    if (n == 0) { free(rank); return 0; }
    if (n == 1) { lens[rank[0].s] = 1; free(rank); return 0; }
    if (n > 256) { free(rank); return -1; }
    /* insertion sort: count descending, symbol ascending */
    for (int i = 1; i < n; i++) {
        or_leaf v = rank[i];
        int j = i - 1;
        while (j >= 0 && (rank[j].c < v.c || (rank[j].c == v.c && rank[j].s > v.s))) { rank[j + 1] = rank[j]; j--; }
        rank[j + 1] = v;
    }
    /* total count of ranks [0, k) */
    uint64_t *head = (uint64_t *)calloc((size_t)n + 1, sizeof(uint64_t));
    for (int i = 0; i < n; i++) head[i + 1] = head[i] + rank[i].c;
    const int64_t full = 2048;                 /* Kraft sum 1 in units of 2^-11 */
    uint64_t best = UINT64_MAX;
    int best_len[4] = {0, 0, 0, 0}, best_end[3] = {0, 0, 0};
    for (int a = 1; a <= 8; a++)
      for (int b = a + 1; b <= 8; b++)
        for (int c = b + 1; c <= 8; c++)
          for (int d = c + 1; d <= 11; d++) {
            int64_t wa = full >> a, wb = full >> b, wc = full >> c, wd = full >> d;
            for (int n1 = 0; n1 <= n; n1++) {
              if (n1 * wa > full) break;
              for (int n2 = 0; n1 + n2 <= n; n2++) {
                int64_t used = n1 * wa + n2 * wb;
                if (used > full) break;
                int64_t left = n - n1 - n2;
                int64_t spare = full - used - left * wd;       /* Kraft room once the rest takes d */
                if (spare < 0) continue;
                int64_t n3 = spare / (wc - wd);
                if (n3 > left) n3 = left;
                int e1 = n1, e2 = n1 + n2, e3 = n1 + n2 + (int)n3;
                uint64_t bits = (uint64_t)a * head[e1] + (uint64_t)b * (head[e2] - head[e1]) +
                                (uint64_t)c * (head[e3] - head[e2]) + (uint64_t)d * (head[n] - head[e3]);
                if (bits < best) {
                  best = bits;
                  best_len[0] = a; best_len[1] = b; best_len[2] = c; best_len[3] = d;
                  best_end[0] = e1; best_end[1] = e2; best_end[2] = e3;
                }
              }
            }
          }
    for (int i = 0; i < n; i++) {
        int g = i < best_end[0] ? 0 : (i < best_end[1] ? 1 : (i < best_end[2] ? 2 : 3));
        lens[rank[i].s] = (uint8_t)best_len[g];
    }
    free(head);
    free(rank);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Canonical code and the decoder's per-length arrays.                  */
/* ------------------------------------------------------------------ */
/* Reading: canonical assignment in the manner of RFC 1951 section 3.2.2:
 * shorter codes are numerically smaller, and codes of one length are
 * consecutive in ascending symbol order.  For each length L (1..11):
 *   count[L]  = number of symbols of length L
 *   first[L]  = the first code of length L
 *   limit[L]  = (first[L] + count[L]) << (11 - L), the 11-bit peek bound
 *   offset[L] = number of symbols with a shorter code
 * and sym_sorted lists the symbols by (length, symbol).  [LW] section
 * "3 . Decode on demand" and the Fig. 3 caption: the decoder finds a code's
 * length by comparing the next 11 stream bits with one bound per length, and
 * finds the symbol at that length's base position plus the code's rank.  Entries at index 0 of the per-length arrays are unused. */
int or_canonical(int n_alpha, const uint8_t *lens, uint16_t *codes,
                 uint16_t *count, uint16_t *first, uint16_t *limit, uint16_t *offset,
                 uint16_t *sym_sorted)
{
    for (int L = 0; L <= OR_MAXLEN; L++) { count[L] = first[L] = limit[L] = offset[L] = 0; }
    for (int s = 0; s < n_alpha; s++) {
        if (lens[s] > OR_MAXLEN) return -1;
        if (lens[s]) count[lens[s]]++;
    }
    uint32_t code = 0;
    uint32_t next_code[OR_MAXLEN + 1];
    next_code[0] = 0;
    for (int L = 1; L <= OR_MAXLEN; L++) {
        code = (code + count[L - 1]) << 1;      /* count[0] is 0 */
        next_code[L] = code;
    }
    for (int L = 1; L <= OR_MAXLEN; L++) first[L] = (uint16_t)next_code[L];
    for (int s = 0; s < n_alpha; s++) {
        codes[s] = 0;
        if (lens[s]) codes[s] = (uint16_t)next_code[lens[s]]++;
    }
    int acc = 0;
    for (int L = 1; L <= OR_MAXLEN; L++) {
        offset[L] = (uint16_t)acc;
        acc += count[L];
        limit[L] = (uint16_t)(((uint32_t)first[L] + count[L]) << (OR_MAXLEN - L));
    }
    int k = 0;
    for (int L = 1; L <= OR_MAXLEN; L++)
        for (int s = 0; s < n_alpha; s++)
            if (lens[s] == L) sym_sorted[k++] = (uint16_t)s;
    return k;
}

/* ------------------------------------------------------------------ */
/* Lane streams and the interleave.                                     */
/* ------------------------------------------------------------------ */
/* Reading ([LW] Fig. 3a and its caption): a lane's codes form a single bit
 * stream cut into 32-bit words; codes are packed MSB-first (bit 31 of a
 * lane's word 0 is its first bit) and the last word is zero-filled.  The
 * words of the 32 lanes alternate so that the j-th words of all lanes sit
 * side by side and one aligned access reads them together:
 * word j of lane l sits at block[32*j + l], every lane being padded with zero
 * words to the tile's longest lane W_t.  tile_off[t] is the word offset of
 * tile t's block (an offset per tile, so each tile decodes independently),
 * tile_off[n_tiles] the total.  lane_bits receives each lane's bit count.
 *
 * With words == NULL only tile_off and lane_bits are filled (sizing pass).
 * Returns the total number of words. */
int64_t or_encode_tiles(int64_t n_tiles, int spl, const uint16_t *syms,
                        const uint8_t *lens, const uint16_t *codes,
                        uint32_t *tile_off, uint32_t *words, uint32_t *lane_bits)
{
    int64_t pos = 0;
    for (int64_t t = 0; t < n_tiles; t++) {
        int64_t nw[OR_LANES];
        int64_t wmax = 0;
        for (int l = 0; l < OR_LANES; l++) {
            const uint16_t *s = syms + (t * OR_LANES + l) * spl;
            int64_t bits = 0;
            for (int k = 0; k < spl; k++) bits += lens[s[k]];
            lane_bits[t * OR_LANES + l] = (uint32_t)bits;
            nw[l] = (bits + 31) / 32;
            if (nw[l] > wmax) wmax = nw[l];
        }
        tile_off[t] = (uint32_t)pos;
        if (words) {
            for (int64_t i = 0; i < 32 * wmax; i++) words[pos + i] = 0;
            for (int l = 0; l < OR_LANES; l++) {
                const uint16_t *s = syms + (t * OR_LANES + l) * spl;
                int64_t bit = 0;            /* bit index within the lane stream */
                for (int k = 0; k < spl; k++) {
                    int len = lens[s[k]];
                    uint32_t c = codes[s[k]];
                    for (int b = len - 1; b >= 0; b--) {   /* MSB of the code first */
                        uint32_t v = (c >> b) & 1u;
                        int64_t j = bit / 32;
                        int within = (int)(bit % 32);
                        if (v) words[pos + 32 * j + l] |= 1u << (31 - within);
                        bit++;
                    }
                }
            }
        }
        pos += 32 * wmax;
    }
    tile_off[n_tiles] = (uint32_t)pos;
    return pos;
}

/* Bit i of lane l's stream in tile block `blk` of `nrow` word rows; bits past
 * the block read as zero. */
static int lane_bit(const uint32_t *blk, int64_t nrow, int l, int64_t i)
{
    int64_t j = i / 32;
    if (j >= nrow) return 0;
    return (int)((blk[32 * j + l] >> (31 - (i % 32))) & 1u);
}

/* Limit-method decode, [LW] section "3 . Decode on demand" and the Fig. 3
 * caption: peek 11 bits, take the shortest length L whose limit exceeds the
 * peek, index the symbol table with offset[L] + (peek >> (11-L)) - first[L],
 * and advance by L.  Returns 0, or -1 if a peek matches no length. */
int or_decode_limit(int64_t n_tiles, int spl, const uint32_t *tile_off, const uint32_t *words,
                    const uint16_t *count, const uint16_t *first, const uint16_t *limit,
                    const uint16_t *offset, const uint16_t *sym_sorted,
                    uint16_t *syms_out, uint32_t *lane_bits_out)
{
    (void)count;
    for (int64_t t = 0; t < n_tiles; t++) {
        const uint32_t *blk = words + tile_off[t];
        int64_t nrow = ((int64_t)tile_off[t + 1] - tile_off[t]) / 32;
        for (int l = 0; l < OR_LANES; l++) {
            int64_t bit = 0;
            uint16_t *out = syms_out + (t * OR_LANES + l) * spl;
            for (int k = 0; k < spl; k++) {
                uint32_t peek = 0;
                for (int b = 0; b < OR_MAXLEN; b++)
                    peek = (peek << 1) | (uint32_t)lane_bit(blk, nrow, l, bit + b);
                int len = 0;
                for (int L = 1; L <= OR_MAXLEN; L++)
                    if (peek < limit[L]) { len = L; break; }
                if (len == 0) return -1;
                uint32_t code = peek >> (OR_MAXLEN - len);
                int idx = (int)offset[len] + (int)code - (int)first[len];
                out[k] = sym_sorted[idx];
                bit += len;
            }
            if (lane_bits_out) lane_bits_out[t * OR_LANES + l] = (uint32_t)bit;
        }
    }
    return 0;
}

/* Independent decode: read one bit at a time, growing (length, code) until it
 * is a code word.  Returns -1 on a length above 11. */
int or_decode_bitwise(int64_t n_tiles, int spl, const uint32_t *tile_off, const uint32_t *words,
                      int n_alpha, const uint8_t *lens, const uint16_t *codes, uint16_t *syms_out)
{
    /* code map: for each length, code -> symbol (or -1) */
    int *map = (int *)malloc(sizeof(int) * (OR_MAXLEN + 1) * 2048);
    for (int i = 0; i < (OR_MAXLEN + 1) * 2048; i++) map[i] = -1;
    for (int s = 0; s < n_alpha; s++)
        if (lens[s]) map[lens[s] * 2048 + codes[s]] = s;
    for (int64_t t = 0; t < n_tiles; t++) {
        const uint32_t *blk = words + tile_off[t];
        int64_t nrow = ((int64_t)tile_off[t + 1] - tile_off[t]) / 32;
        for (int l = 0; l < OR_LANES; l++) {
            int64_t bit = 0;
            uint16_t *out = syms_out + (t * OR_LANES + l) * spl;
            for (int k = 0; k < spl; k++) {
                int len = 0;
                uint32_t code = 0;
                int sym = -1;
                while (sym < 0) {
                    code = (code << 1) | (uint32_t)lane_bit(blk, nrow, l, bit);
                    bit++;
                    len++;
                    if (len > OR_MAXLEN) { free(map); return -1; }
                    sym = map[len * 2048 + code];
                }
                out[k] = (uint16_t)sym;
            }
        }
    }
    free(map);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Scales and the GEMV.                                                 */
/* ------------------------------------------------------------------ */

/* Exact fp16 -> double. */
double or_half_to_double(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* double -> fp16 bits, round to nearest with ties to even (IEEE 754
 * binary16), the rounding the activations between the MLP projections get.
 * Worked from the binary expansion: a = f * 2^e, f in [0.5, 1), keeps an
 * 11-bit significand; below 2^-14 the grid is multiples of 2^-24; from
 * 65520 (halfway to 2^16) on the result is infinity. */
uint16_t or_double_to_half(double v)
{
    const uint16_t s = signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (isnan(v)) return 0x7E00u;
    if (a >= 65520.0) return (uint16_t)(s | 0x7C00u);
    if (a < ldexp(1.0, -14)) {
        const double q = nearbyint(ldexp(a, 24));     /* exact scaling, then ties to even */
        return (uint16_t)(s | (uint16_t)q);           /* q == 1024 is the smallest normal */
    }
    int e;
    const double f = frexp(a, &e);
    double q = nearbyint(ldexp(f, 11));                /* significand in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        e += 1;
    }
    const int E = e - 1 + 15;
    if (E >= 31) return (uint16_t)(s | 0x7C00u);
    return (uint16_t)(s | (uint16_t)(E << 10) | (uint16_t)((int)q - 1024));
}

/* SwiGLU activation of an MLP ([UW] "Overlapping Work Across Transformer
 * Layers": the down projection consumes gate, activation and up; "Measured
 * Results": SwiGLU architectures): h = fp16(silu(g) * u) with
 * silu(z) = z / (1 + e^-z), in double, rounded once. */
void or_swiglu(int64_t n, const double *g, const double *u, uint16_t *h)
{
    for (int64_t i = 0; i < n; i++) h[i] = or_double_to_half(g[i] / (1.0 + exp(-g[i])) * u[i]);
}

/* Exact bf16 -> double. */
double or_bf16_to_double(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 255, m = b & 127;
    double v;
    if (e == 0) v = ldexp((double)m, -133);
    else if (e == 255) v = m ? NAN : INFINITY;
    else v = ldexp((double)(128 + m), e - 134);
    return s ? -v : v;
}

/* Reading of the rule that scales and minimums are kept in llama.cpp's raw
 * form ([LW] section 2), under the
 * synthetic workloads: one fp16 (d, m) per 256-weight super-block, a
 * super-block being one tile row.  dm[t][i] = d | m << 16 for tile row i. */
void or_pack_dm(int64_t rows, int64_t cols, const uint16_t *d, const uint16_t *m, uint32_t *dm)
{
    int64_t nrb = rows / OR_TILE_ROWS, ncb = cols / OR_TILE_COLS;
    for (int64_t rb = 0; rb < nrb; rb++)
        for (int64_t cb = 0; cb < ncb; cb++)
            for (int i = 0; i < OR_TILE_ROWS; i++) {
                int64_t r = rb * OR_TILE_ROWS + i;
                dm[(rb * ncb + cb) * OR_TILE_ROWS + i] =
                    (uint32_t)d[r * ncb + cb] | ((uint32_t)m[r * ncb + cb] << 16);
            }
}

/* y[b][r] = sum_c (d[r][c/256] * q[r][c] - m[r][c/256]) * x[b][c], in double,
 * fp16 inputs converted exactly ([SDB] IV-A: grouped storage with a scale and
 * a zero per group; dequantisation w = d*q - m per 256-weight super-block).
 * Rows listed in `row_list` (n_list of them) only, or all rows if NULL;
 * y is [batch][n_list or rows]. */
void or_gemv_q(int64_t rows, int64_t cols, const uint8_t *q, const uint16_t *d,
               const uint16_t *m, const uint16_t *x, int batch,
               const int64_t *row_list, int64_t n_list, double *y)
{
    int64_t ncb = cols / OR_TILE_COLS;
    int64_t nr = row_list ? n_list : rows;
    for (int b = 0; b < batch; b++)
        for (int64_t i = 0; i < nr; i++) {
            int64_t r = row_list ? row_list[i] : i;
            double acc = 0.0;
            for (int64_t c = 0; c < cols; c++) {
                double dd = or_half_to_double(d[r * ncb + c / OR_TILE_COLS]);
                double mm = or_half_to_double(m[r * ncb + c / OR_TILE_COLS]);
                double w = dd * (double)q[r * cols + c] - mm;
                acc += w * or_half_to_double(x[(int64_t)b * cols + c]);
            }
            y[(int64_t)b * nr + i] = acc;
        }
}

/* Dense bf16 GEMV in double (bf16 -> double is exact). */
void or_gemv_bf16(int64_t rows, int64_t cols, const uint16_t *w, const uint16_t *x, int batch,
                  const int64_t *row_list, int64_t n_list, double *y)
{
    int64_t nr = row_list ? n_list : rows;
    for (int b = 0; b < batch; b++)
        for (int64_t i = 0; i < nr; i++) {
            int64_t r = row_list ? row_list[i] : i;
            double acc = 0.0;
            for (int64_t c = 0; c < cols; c++)
                acc += or_bf16_to_double(w[r * cols + c]) * or_bf16_to_double(x[(int64_t)b * cols + c]);
            y[(int64_t)b * nr + i] = acc;
        }
}

/* ------------------------------------------------------------------ */
/* BF16 exponent coding ([UW]).                                         */
/* ------------------------------------------------------------------ */
/* Field split: sign 1 bit, exponent 8 bits, mantissa 7 bits.  Only the
 * exponent is entropy coded; sign and mantissa are kept raw as one byte
 * sm = sign << 7 | mantissa. */
uint8_t or_bf16_exponent(uint16_t w) { return (uint8_t)((w >> 7) & 0xFF); }
uint8_t or_bf16_sm(uint16_t w) { return (uint8_t)(((w >> 15) << 7) | (w & 0x7F)); }
uint16_t or_bf16_join(uint8_t sm, uint8_t e)
{
    return (uint16_t)(((uint16_t)(sm >> 7) << 15) | ((uint16_t)e << 7) | (sm & 0x7F));
}

/* Palette: the matrix's 16 most frequent exponents ([UW]: in trained bf16
 * weights they account for more than 99 % of the values), ordered by (count descending,
 * exponent ascending) so index 0 is the most frequent.  Returns the number
 * of distinct exponents placed (<= 16); unused entries are 0. */
int or_bf16_palette(int64_t n, const uint16_t *w, uint8_t *palette)
{
    uint64_t cnt[256];
    int used[256];
    for (int e = 0; e < 256; e++) { cnt[e] = 0; used[e] = 0; }
    for (int64_t i = 0; i < n; i++) cnt[or_bf16_exponent(w[i])]++;
    int k = 0;
    for (; k < 16; k++) {
        int best = -1;
        for (int e = 0; e < 256; e++) {
            if (used[e] || cnt[e] == 0) continue;
            if (best < 0 || cnt[e] > cnt[best]) best = e;   /* ascending e wins ties */
        }
        if (best < 0) break;
        used[best] = 1;
        palette[k] = (uint8_t)best;
    }
    for (int j = k; j < 16; j++) palette[j] = 0;
    return k;
}

/* Verbatim segments ([UW]: a 64-weight row whose exponents are not all in
 * the palette is kept uncompressed as a whole).  Reading:
 * segments are 64-aligned runs along a matrix row, four per tile row.
 * vb_bits[t][8] bit (4*i + s) marks segment s of tile row i; vb_start[t] is
 * the number of verbatim segments in tiles before t; `verbatim` receives the
 * raw bf16 values of each segment, tiles in order, then tile rows, then
 * segments.  Returns the number of verbatim segments (pass verbatim = NULL to
 * count only). */
int64_t or_bf16_verbatim(int64_t rows, int64_t cols, const uint16_t *w, const uint8_t *palette,
                         int n_pal, uint32_t *vb_bits, uint32_t *vb_start, uint16_t *verbatim)
{
    int64_t nrb = rows / OR_TILE_ROWS, ncb = cols / OR_TILE_COLS;
    int inpal[256];
    for (int e = 0; e < 256; e++) inpal[e] = 0;
    for (int k = 0; k < n_pal; k++) inpal[palette[k]] = 1;
    int64_t nv = 0;
    for (int64_t rb = 0; rb < nrb; rb++)
        for (int64_t cb = 0; cb < ncb; cb++) {
            int64_t t = rb * ncb + cb;
            vb_start[t] = (uint32_t)nv;
            for (int j = 0; j < 8; j++) vb_bits[t * 8 + j] = 0;
            for (int i = 0; i < OR_TILE_ROWS; i++)
                for (int s = 0; s < 4; s++) {
                    const uint16_t *seg = w + (rb * OR_TILE_ROWS + i) * cols + cb * OR_TILE_COLS + 64 * s;
                    int out = 0;
                    for (int c = 0; c < 64; c++)
                        if (!inpal[or_bf16_exponent(seg[c])]) out = 1;
                    if (out) {
                        int bit = 4 * i + s;
                        vb_bits[t * 8 + bit / 32] |= 1u << (bit % 32);
                        if (verbatim) memcpy(verbatim + nv * 64, seg, 64 * sizeof(uint16_t));
                        nv++;
                    }
                }
        }
    vb_start[nrb * ncb] = (uint32_t)nv;
    return nv;
}

/* Exponent symbols in the lane order of or_symbolise_q (singles, 512 per
 * lane): the palette index of the exponent, or 0 for every weight of a
 * verbatim segment (a placeholder that keeps all lanes at 512 symbols). */
void or_bf16_symbolise(int64_t rows, int64_t cols, const uint16_t *w, const uint8_t *palette,
                       int n_pal, const uint32_t *vb_bits, uint16_t *syms)
{
    int64_t nrb = rows / OR_TILE_ROWS, ncb = cols / OR_TILE_COLS;
    int idx_of[256];
    for (int e = 0; e < 256; e++) idx_of[e] = -1;
    for (int k = 0; k < n_pal; k++) idx_of[palette[k]] = k;
    for (int64_t rb = 0; rb < nrb; rb++)
        for (int64_t cb = 0; cb < ncb; cb++) {
            int64_t t = rb * ncb + cb;
            for (int l = 0; l < OR_LANES; l++) {
                uint16_t *out = syms + (t * OR_LANES + l) * 512;
                int k = 0;
                for (int half = 0; half < 2; half++) {
                    int i = 2 * l + half;
                    const uint16_t *row = w + (rb * OR_TILE_ROWS + i) * cols + cb * OR_TILE_COLS;
                    for (int c = 0; c < OR_TILE_COLS; c++) {
                        int bit = 4 * i + c / 64;
                        int verb = (vb_bits[t * 8 + bit / 32] >> (bit % 32)) & 1;
                        out[k++] = verb ? 0 : (uint16_t)idx_of[or_bf16_exponent(row[c])];
                    }
                }
            }
        }
}

/* Raw sign+mantissa bytes, lane-interleaved like the Huffman words.
 * Reading (the pages only say sign and mantissa stay untouched): tile t owns
 * 4096 words; word (p*64 + g)*32 + l holds, in bytes 0..3, the sm bytes of
 * tile row 2l + p, columns 4g .. 4g+3.  So lane l reads its own row's bytes
 * in decode order with one coalesced 128-byte read per 32 lanes. */
void or_bf16_pack_sm(int64_t rows, int64_t cols, const uint16_t *w, uint32_t *sm)
{
    int64_t nrb = rows / OR_TILE_ROWS, ncb = cols / OR_TILE_COLS;
    for (int64_t rb = 0; rb < nrb; rb++)
        for (int64_t cb = 0; cb < ncb; cb++) {
            int64_t t = rb * ncb + cb;
            uint32_t *blk = sm + t * 4096;
            for (int p = 0; p < 2; p++)
                for (int g = 0; g < 64; g++)
                    for (int l = 0; l < OR_LANES; l++) {
                        const uint16_t *row = w + (rb * OR_TILE_ROWS + 2 * l + p) * cols + cb * OR_TILE_COLS;
                        uint32_t v = 0;
                        for (int b = 0; b < 4; b++)
                            v |= (uint32_t)or_bf16_sm(row[4 * g + b]) << (8 * b);
                        blk[(p * 64 + g) * 32 + l] = v;
                    }
        }
}

/* Rebuild the bf16 matrix from decoded exponent symbols, the sm words, the
 * palette and the verbatim store. */
void or_bf16_reconstruct(int64_t rows, int64_t cols, const uint16_t *syms, const uint32_t *sm,
                         const uint8_t *palette, const uint32_t *vb_bits, const uint32_t *vb_start,
                         const uint16_t *verbatim, uint16_t *w_out)
{
    int64_t nrb = rows / OR_TILE_ROWS, ncb = cols / OR_TILE_COLS;
    for (int64_t rb = 0; rb < nrb; rb++)
        for (int64_t cb = 0; cb < ncb; cb++) {
            int64_t t = rb * ncb + cb;
            const uint32_t *blk = sm + t * 4096;
            /* ordinal of each verbatim segment inside the tile */
            int64_t vord = vb_start[t];
            int64_t seg_index[256];
            for (int bit = 0; bit < 256; bit++) {
                if ((vb_bits[t * 8 + bit / 32] >> (bit % 32)) & 1) seg_index[bit] = vord++;
                else seg_index[bit] = -1;
            }
            for (int l = 0; l < OR_LANES; l++) {
                const uint16_t *s = syms + (t * OR_LANES + l) * 512;
                for (int p = 0; p < 2; p++) {
                    int i = 2 * l + p;
                    uint16_t *row = w_out + (rb * OR_TILE_ROWS + i) * cols + cb * OR_TILE_COLS;
                    for (int c = 0; c < OR_TILE_COLS; c++) {
                        int bit = 4 * i + c / 64;
                        if (seg_index[bit] >= 0) {
                            row[c] = verbatim[seg_index[bit] * 64 + (c % 64)];
                        } else {
                            uint8_t smb = (uint8_t)(blk[(p * 64 + c / 4) * 32 + l] >> (8 * (c % 4)));
                            row[c] = or_bf16_join(smb, palette[s[p * 256 + c]]);
                        }
                    }
                }
            }
        }
}

/* ------------------------------------------------------------------------
 * Tile-skipping fixed-width GEMV ([SDB] IV-A storage, IV-B layout, IV-C
 * kernel and traffic ledger).
 *
 * Storage: b-bit codes (b in {2, 4, 8}), floor(32/b) = 32/b per 32-bit word,
 * the weight at position i of a word in bits b*i .. b*i+b-1 (low bits first:
 * the reading of "packed into 32-bit words" used here).  Groups of 256
 * columns carry an fp16 scale d and zero m, w = d*q - m (the super-block of
 * the coded path, so all paths share the same d, m).
 * Layout: words[t][j][r] with t the tile of B_N = 64 consecutive rows, j the
 * word column (0 .. WPR-1, WPR = cols / (32/b)) and r the row within the
 * tile; scales dm[t][g][r] = d | m << 16 for the 256-column group g.
 */
#define OR_SKIP_BN 64

void or_skip_pack(int64_t rows, int64_t cols, int bits, const uint8_t *q, const uint16_t *d,
                  const uint16_t *m, uint32_t *words, uint32_t *dm)
{
    int64_t per = 32 / bits, wpr = cols / per, ng = cols / OR_TILE_COLS;
    for (int64_t r = 0; r < rows; r++) {
        int64_t t = r / OR_SKIP_BN, rr = r % OR_SKIP_BN;
        for (int64_t j = 0; j < wpr; j++) {
            uint32_t w = 0;
            for (int64_t i = 0; i < per; i++)
                w |= (uint32_t)q[r * cols + j * per + i] << (bits * i);
            words[(t * wpr + j) * OR_SKIP_BN + rr] = w;
        }
        for (int64_t g = 0; g < ng; g++)
            dm[(t * ng + g) * OR_SKIP_BN + rr] = (uint32_t)d[r * ng + g] | ((uint32_t)m[r * ng + g] << 16);
    }
}

/* y[b][r] in double for the rows of every tile in the list, read back from
 * the packed words and scales; rows of other tiles are not written.  A list
 * entry outside 0 .. n_tiles-1 names no tile and is skipped (a repeated entry
 * writes the same values again). */
void or_skip_gemv(int64_t rows, int64_t cols, int bits, const uint32_t *words, const uint32_t *dm,
                  const int32_t *tiles, int64_t n_list, const uint16_t *x, int batch, double *y)
{
    int64_t per = 32 / bits, wpr = cols / per, ng = cols / OR_TILE_COLS, nt = rows / OR_SKIP_BN;
    uint32_t mask = (1u << bits) - 1u;
    for (int64_t k = 0; k < n_list; k++) {
        int64_t t = tiles[k];
        if (t < 0 || t >= nt) continue;
        for (int b = 0; b < batch; b++)
            for (int64_t rr = 0; rr < OR_SKIP_BN; rr++) {
                double acc = 0.0;
                for (int64_t j = 0; j < wpr; j++) {
                    uint32_t w = words[(t * wpr + j) * OR_SKIP_BN + rr];
                    for (int64_t i = 0; i < per; i++) {
                        int64_t c = j * per + i;
                        uint32_t sc = dm[(t * ng + c / OR_TILE_COLS) * OR_SKIP_BN + rr];
                        double q = (double)((w >> (bits * i)) & mask);
                        double wt = or_half_to_double((uint16_t)(sc & 0xFFFF)) * q -
                                    or_half_to_double((uint16_t)(sc >> 16));
                        acc += wt * or_half_to_double(x[(int64_t)b * cols + c]);
                    }
                }
                y[(int64_t)b * rows + t * OR_SKIP_BN + rr] = acc;
            }
    }
}

/* Traffic ledger of one call with n_active listed tiles ([SDB] IV-C: the
 * words touched are exactly n_active * WPR * B_N).  out[0] words, out[1]
 * word bytes, out[2] scale bytes, out[3] activation bytes, out[4] output
 * bytes, out[5] their sum. */
void or_skip_ledger(int64_t cols, int bits, int64_t n_active, int batch, uint64_t out[6])
{
    uint64_t wpr = (uint64_t)(cols / (32 / bits));
    out[0] = (uint64_t)n_active * wpr * OR_SKIP_BN;
    out[1] = 4 * out[0];
    out[2] = (uint64_t)n_active * (uint64_t)(cols / OR_TILE_COLS) * OR_SKIP_BN * 4;
    out[3] = (uint64_t)batch * (uint64_t)cols * 2;
    out[4] = (uint64_t)batch * (uint64_t)n_active * OR_SKIP_BN * 4;
    out[5] = out[1] + out[2] + out[3] + out[4];
}

/* ------------------------------------------------------------------------
 * rANS lane coder (decode-cost ablation).  [LW] section "Decoder hardware",
 * paragraph on Huffman against rANS: at equal rate an rANS decoder is never
 * smaller in bits and needs more area.  The pages give no rANS format; the
 * readings here:
 *   - one frequency table per matrix, scaled to M = 2^11 = 2048 (so the
 *     rarest symbol costs at most 11 bits, the Huffman code-length limit);
 *   - one stream per tile row (64 per tile), the row's symbols in column
 *     order (4-bit codes in pairs, low nibble the even column; 6-bit codes
 *     singly), or, as an option, two per row (128 per tile), one per half
 *     of the row's columns: stream h*64 + r holds half h of row r;
 *   - 32-bit state x in [L, 2^16 L) with L = 2^16, renormalised 16 bits at a
 *     time; a stream is its final encoder state followed by its 16-bit
 *     chunks in decoding order;
 *   - a tile block of ns streams is the ns head states (word s for stream
 *     s), then the chunks as 16-bit units, chunk k of stream s at unit
 *     ns*k + s (little-endian: unit h is the low half of the block's word
 *     ns + h/2 when h is even), every stream zero-padded to the tile's
 *     chunk count K_t, rounded up to even, so a block is ns + ns*K_t/2
 *     words.
 * ------------------------------------------------------------------------ */
#define OR_RANS_PB 11
#define OR_RANS_M (1u << OR_RANS_PB)
#define OR_RANS_L (1u << 16)

/* Frequencies f[s] summing to M: f = 0 for an absent symbol, else
 * max(1, round-half-up(count * M / total)); then, while the sum exceeds M,
 * take 1 from the largest f above 1 (ties: the smallest symbol), and while
 * it falls short, give 1 to the largest f (ties: the smallest symbol).
 * cum[s] = sum of f over the symbols below s.  Returns the number of used
 * symbols, or -1 if the sum cannot be fixed (more than M used symbols). */
int or_rans_freqs(int n_alpha, const uint64_t *counts, uint16_t *f, uint16_t *cum)
{
    uint64_t total = 0;
    int used = 0;
    for (int s = 0; s < n_alpha; s++) { total += counts[s]; if (counts[s]) used++; }
    int64_t sum = 0;
    for (int s = 0; s < n_alpha; s++) {
        if (!counts[s]) { f[s] = 0; continue; }
        uint64_t v = (2u * counts[s] * OR_RANS_M + total) / (2u * total);
        f[s] = (uint16_t)(v < 1 ? 1 : v);
        sum += f[s];
    }
    while (sum != (int64_t)OR_RANS_M && used > 0) {
        int pick = -1;
        for (int s = 0; s < n_alpha; s++) {
            if (!f[s] || (sum > (int64_t)OR_RANS_M && f[s] <= 1)) continue;
            if (pick < 0 || f[s] > f[pick]) pick = s;
        }
        if (pick < 0) return -1;
        if (sum > (int64_t)OR_RANS_M) { f[pick]--; sum--; }
        else { f[pick]++; sum++; }
    }
    uint32_t c = 0;
    for (int s = 0; s < n_alpha; s++) { cum[s] = (uint16_t)c; c += f[s]; }
    return used;
}

/* Symbols of the 64 row streams of every tile: stream (t, r) holds tile row
 * r, spr symbols (128 pairs or 256 singles), at syms[(t*64 + r)*spr + i]. */
void or_rans_symbolise(int kind, int64_t rows, int64_t cols, const uint8_t *q, uint16_t *syms)
{
    int64_t ncb = cols / OR_TILE_COLS, nt = (rows / OR_TILE_ROWS) * ncb;
    int spr = kind == OR_Q4 ? 128 : 256;
    for (int64_t t = 0; t < nt; t++)
        for (int r = 0; r < 64; r++) {
            const uint8_t *row = q + ((t / ncb) * 64 + r) * cols + (t % ncb) * OR_TILE_COLS;
            uint16_t *o = syms + (t * 64 + r) * spr;
            for (int i = 0; i < spr; i++)
                o[i] = kind == OR_Q4 ? (uint16_t)(row[2 * i] | (row[2 * i + 1] << 4)) : row[i];
        }
}

/* Encode one stream of n symbols: *state receives the final encoder state,
 * chunks[0 .. returned count) the 16-bit chunks in decoding order (at most
 * one per symbol, so chunks holds n entries).  Encoding runs from the last
 * symbol to the first; before each symbol the state is brought below
 * 2^21 f[s] by emitting its low 16 bits, which keeps the coded state below
 * 2^32. */
int or_rans_encode_stream(const uint16_t *s, int n, const uint16_t *f, const uint16_t *cum,
                          uint32_t *state, uint16_t *chunks)
{
    uint32_t x = OR_RANS_L;
    int k = 0;                                     /* chunks emitted, in encoding order */
    for (int i = n - 1; i >= 0; i--) {
        uint32_t fs = f[s[i]];
        uint64_t xmax = ((uint64_t)(OR_RANS_L >> OR_RANS_PB) << 16) * fs;
        while ((uint64_t)x >= xmax) { chunks[k++] = (uint16_t)(x & 0xFFFF); x >>= 16; }
        x = (x / fs) * OR_RANS_M + (x % fs) + cum[s[i]];
    }
    *state = x;
    for (int a = 0, b = k - 1; a < b; a++, b--) {  /* decoding order = reverse of emission */
        uint16_t tmp = chunks[a]; chunks[a] = chunks[b]; chunks[b] = tmp;
    }
    return k;
}

/* Encode all tiles: ns streams of sps symbols per tile, stream (t, s) at
 * syms[(t*ns + s)*sps]; tile_off[nt+1] (word offsets) and, unless words is
 * NULL (sizing pass), the blocks: the ns head states (word s for stream s),
 * then chunk k of stream s at 16-bit unit ns*k + s, zero-padded to the
 * tile's chunk count rounded up to even.  Returns the total word count. */
int64_t or_rans_encode_tiles(int64_t nt, int ns, int sps, const uint16_t *syms, const uint16_t *f,
                             const uint16_t *cum, uint32_t *tile_off, uint32_t *words)
{
    uint16_t *ch = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)sps * (size_t)ns);
    int *nk = (int *)malloc(sizeof(int) * (size_t)ns);
    uint32_t *st = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)ns);
    int64_t pos = 0;
    for (int64_t t = 0; t < nt; t++) {
        tile_off[t] = (uint32_t)pos;
        int kmax = 0;
        for (int r = 0; r < ns; r++) {
            nk[r] = or_rans_encode_stream(syms + (t * ns + r) * sps, sps, f, cum, &st[r], ch + (size_t)r * sps);
            if (nk[r] > kmax) kmax = nk[r];
        }
        int kt = (kmax + 1) & ~1;
        int64_t nw = ns + (int64_t)ns * kt / 2;
        if (words) {
            uint32_t *blk = words + pos;
            for (int64_t i = 0; i < nw; i++) blk[i] = 0;
            for (int r = 0; r < ns; r++) {
                blk[r] = st[r];
                for (int k = 0; k < nk[r]; k++) {
                    int64_t h = (int64_t)ns * k + r;            /* 16-bit unit in the chunk area */
                    blk[ns + h / 2] |= (uint32_t)ch[(size_t)r * sps + k] << (16 * (h & 1));
                }
            }
        }
        pos += nw;
    }
    tile_off[nt] = (uint32_t)pos;
    free(ch);
    free(nk);
    free(st);
    return pos;
}

/* Decode one stream of n symbols from its head state and its chunks, chunk
 * k at chunks[stride * k] (nchunks of them).  A symbol's slot range is found
 * by a plain search over the cumulative frequencies.  The stream must end in
 * state L having read only its own chunks.  Returns 0, or -1 otherwise. */
int or_rans_decode_stream(uint32_t state, const uint16_t *chunks, int64_t stride, int64_t nchunks, int n,
                          int n_alpha, const uint16_t *f, const uint16_t *cum, uint16_t *out)
{
    uint32_t x = state;
    int64_t k = 0;
    for (int i = 0; i < n; i++) {
        uint32_t slot = x & (OR_RANS_M - 1);
        int s = -1;
        for (int c = 0; c < n_alpha; c++)
            if (f[c] && cum[c] <= slot && slot < (uint32_t)cum[c] + f[c]) { s = c; break; }
        if (s < 0) return -1;
        out[i] = (uint16_t)s;
        x = f[s] * (x >> OR_RANS_PB) + slot - cum[s];
        while (x < OR_RANS_L) {
            if (k >= nchunks) return -1;
            x = (x << 16) | chunks[stride * k];
            k++;
        }
    }
    return x == OR_RANS_L ? 0 : -1;
}

/* Decode all tiles back to symbols (the layout of or_rans_encode_tiles).
 * Returns 0, or -1 if any stream fails.  The chunk area is read through a
 * 16-bit view of the little-endian words. */
int or_rans_decode_tiles(int64_t nt, int ns, int sps, int n_alpha, const uint16_t *f, const uint16_t *cum,
                         const uint32_t *tile_off, const uint32_t *words, uint16_t *syms)
{
    for (int64_t t = 0; t < nt; t++) {
        const uint32_t *blk = words + tile_off[t];
        int64_t nw = (int64_t)tile_off[t + 1] - tile_off[t];
        if (nw < ns || (nw - ns) % (ns / 2)) return -1;
        int64_t kt = (nw - ns) / (ns / 2);
        const uint16_t *area = (const uint16_t *)(blk + ns);
        for (int r = 0; r < ns; r++)
            if (or_rans_decode_stream(blk[r], area + r, ns, kt, sps, n_alpha, f, cum, syms + (t * ns + r) * sps))
                return -1;
    }
    return 0;
}
