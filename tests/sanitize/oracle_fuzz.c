/* Host-only driver for an AddressSanitizer / UndefinedBehaviorSanitizer build
 * of the oracle (oracle/oracle.c): code lengths of random histograms (the
 * optimal and the compact code), canonical tables, encode and both decoders
 * on random symbol streams, decoding of random words under incomplete codes,
 * and the rANS coder on random streams and on corrupted chunks.  The
 * sanitizers abort the process on any memory error or undefined behaviour.
 * Usage: oracle_fuzz [rounds] */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int or_package_merge(int n_alpha, const uint64_t *counts, int L, uint8_t *lens);
int or_compact_lengths(int n_alpha, const uint64_t *counts, uint8_t *lens);
int or_canonical(int n_alpha, const uint8_t *lens, uint16_t *codes, uint16_t *count, uint16_t *first,
                 uint16_t *limit, uint16_t *offset, uint16_t *sym_sorted);
int64_t or_encode_tiles(int64_t n_tiles, int spl, const uint16_t *syms, const uint8_t *lens, const uint16_t *codes,
                        uint32_t *tile_off, uint32_t *words, uint32_t *lane_bits);
int or_decode_limit(int64_t n_tiles, int spl, const uint32_t *tile_off, const uint32_t *words,
                    const uint16_t *count, const uint16_t *first, const uint16_t *limit, const uint16_t *offset,
                    const uint16_t *sym_sorted, uint16_t *syms_out, uint32_t *lane_bits_out);
int or_decode_bitwise(int64_t n_tiles, int spl, const uint32_t *tile_off, const uint32_t *words, int n_alpha,
                      const uint8_t *lens, const uint16_t *codes, uint16_t *syms_out);
int or_rans_freqs(int n_alpha, const uint64_t *counts, uint16_t *f, uint16_t *cum);
int or_rans_encode_stream(const uint16_t *s, int n, const uint16_t *f, const uint16_t *cum, uint32_t *state,
                          uint16_t *chunks);
int or_rans_decode_stream(uint32_t state, const uint16_t *chunks, int64_t stride, int64_t nchunks, int n,
                          int n_alpha, const uint16_t *f, const uint16_t *cum, uint16_t *out);

static uint64_t s_rng = 88172645463325252ull;
static uint64_t rnd(void)
{
    s_rng ^= s_rng << 13;
    s_rng ^= s_rng >> 7;
    s_rng ^= s_rng << 17;
    return s_rng;
}

static int fails = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);        \
            fails++;                                                              \
        }                                                                         \
    } while (0)

int main(int argc, char **argv)
{
    const int rounds = argc > 1 ? atoi(argv[1]) : 300;
    const int spl = 256, n_tiles = 2;
    for (int r = 0; r < rounds; r++) {
        const int n_alpha = (r % 3 == 0) ? 16 : (r % 3 == 1) ? 64 : 256;
        uint64_t counts[256];
        const int n_used = 1 + (int)(rnd() % (uint64_t)n_alpha);
        memset(counts, 0, sizeof(counts));
        for (int i = 0; i < n_used; i++) counts[rnd() % (uint64_t)n_alpha] += 1 + rnd() % ((r & 1) ? 1000000 : 7);
        uint8_t lens[256];
        const int compact = r & 4;
        const int rc = compact ? or_compact_lengths(n_alpha, counts, lens) : or_package_merge(n_alpha, counts, 11, lens);
        CHECK(rc == 0);
        uint16_t codes[256], count[12], first[12], limit[12], offset[12], sym_sorted[256];
        const int n_sym = or_canonical(n_alpha, lens, codes, count, first, limit, offset, sym_sorted);
        CHECK(n_sym >= 1);
        /* symbols drawn from the coded ones */
        int used[256], nu = 0;
        for (int s = 0; s < n_alpha; s++)
            if (lens[s]) used[nu++] = s;
        const int64_t nsym = (int64_t)n_tiles * 32 * spl;
        uint16_t *syms = malloc(sizeof(uint16_t) * (size_t)nsym), *back = malloc(sizeof(uint16_t) * (size_t)nsym);
        for (int64_t i = 0; i < nsym; i++) syms[i] = (uint16_t)used[rnd() % (uint64_t)nu];
        uint32_t tile_off[3], lane_bits[64], lane_bits2[64];
        const int64_t nw = or_encode_tiles(n_tiles, spl, syms, lens, codes, tile_off, NULL, lane_bits);
        CHECK(nw > 0);
        uint32_t *words = malloc(sizeof(uint32_t) * (size_t)nw);
        CHECK(or_encode_tiles(n_tiles, spl, syms, lens, codes, tile_off, words, lane_bits) == nw);
        CHECK(or_decode_limit(n_tiles, spl, tile_off, words, count, first, limit, offset, sym_sorted, back,
                              lane_bits2) == 0);
        CHECK(memcmp(syms, back, sizeof(uint16_t) * (size_t)nsym) == 0);
        CHECK(or_decode_bitwise(n_tiles, spl, tile_off, words, n_alpha, lens, codes, back) == 0);
        CHECK(memcmp(syms, back, sizeof(uint16_t) * (size_t)nsym) == 0);
        /* random words: a decoder either finishes or reports an unmatched peek */
        for (int64_t i = 0; i < nw; i++) words[i] = (uint32_t)rnd();
        (void)or_decode_limit(n_tiles, spl, tile_off, words, count, first, limit, offset, sym_sorted, back, NULL);
        (void)or_decode_bitwise(n_tiles, spl, tile_off, words, n_alpha, lens, codes, back);
        free(words);
        /* rANS: random stream, then corrupted chunks */
        uint16_t f[256], cum[256];
        if (or_rans_freqs(n_alpha, counts, f, cum) == 0) {
            const int n = 1 + (int)(rnd() % 600);
            uint16_t *s = malloc(sizeof(uint16_t) * (size_t)n), *o = malloc(sizeof(uint16_t) * (size_t)n);
            uint16_t *ch = malloc(sizeof(uint16_t) * (size_t)n);
            int un = 0, ru[256];
            for (int a = 0; a < n_alpha; a++)
                if (f[a]) ru[un++] = a;
            for (int i = 0; i < n; i++) s[i] = (uint16_t)ru[rnd() % (uint64_t)un];
            uint32_t st = 0;
            const int k = or_rans_encode_stream(s, n, f, cum, &st, ch);
            CHECK(k >= 0 && k <= n);
            CHECK(or_rans_decode_stream(st, ch, 1, k, n, n_alpha, f, cum, o) == 0);
            CHECK(memcmp(s, o, sizeof(uint16_t) * (size_t)n) == 0);
            for (int i = 0; i < k; i++) ch[i] = (uint16_t)rnd();
            (void)or_rans_decode_stream((uint32_t)rnd(), ch, 1, k, n, n_alpha, f, cum, o);
            free(s);
            free(o);
            free(ch);
        }
        free(syms);
        free(back);
    }
    printf("oracle_fuzz: %d rounds, %d failed checks\n", rounds, fails);
    return fails ? 1 : 0;
}
