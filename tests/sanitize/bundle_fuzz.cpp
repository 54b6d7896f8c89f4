// Host-only driver for an AddressSanitizer / UndefinedBehaviorSanitizer build
// of the bundle builder (decode_gemv_amd/csrc/bundle.cpp): builds bundles of
// every kind and code, then hands lw_bundle_load thousands of corrupted
// images (flipped bytes anywhere, header fields set to extreme values,
// region offsets and sizes moved, truncations) and the builders' argument
// errors.  Every call must return a status; the sanitizers abort the process
// on any out-of-bounds access, overflow or other undefined behaviour.
// Usage: bundle_fuzz [iterations per image]
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "lw.h"

static std::mt19937_64 rng(12345);

static int fails = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            fails++;                                                    \
        }                                                               \
    } while (0)

static std::vector<uint8_t> image_of(lw_bundle *b)
{
    const void *p = nullptr;
    size_t n = 0;
    CHECK(lw_bundle_image(b, &p, &n) == LW_OK);
    const uint8_t *u = static_cast<const uint8_t *>(p);
    return std::vector<uint8_t>(u, u + n);
}

static void exercise(const std::vector<uint8_t> &img)
{
    lw_bundle *b = nullptr;
    lw_status st = lw_bundle_load(img.data(), img.size(), &b);
    if (st == LW_OK) {
        lw_bundle_info info;
        CHECK(lw_bundle_get_info(b, &info) == LW_OK);
        CHECK(lw_bundle_validate(b) == LW_OK);
        for (int r = 0; r < LW_REG_COUNT; r++) {
            const void *p = nullptr;
            size_t n = 0;
            lw_bundle_region(b, r, &p, &n);
        }
        lw_bundle_free(b);
    } else {
        CHECK(b == nullptr);
        CHECK(lw_last_error() != nullptr);
    }
}

static void fuzz_image(const std::vector<uint8_t> &base, int iters)
{
    exercise(base);
    std::uniform_int_distribution<size_t> pos(0, base.size() - 1);
    std::uniform_int_distribution<int> byte(0, 255);
    for (int it = 0; it < iters; it++) {
        std::vector<uint8_t> img = base;
        const int mode = it % 6;
        if (mode == 0) {                       // a few random bytes anywhere
            for (int k = 0; k < 1 + it % 4; k++) img[pos(rng)] ^= (uint8_t)(1 + byte(rng) % 255);
        } else if (mode == 1) {                // header bytes
            for (int k = 0; k < 1 + it % 3; k++) img[rng() % 512] = (uint8_t)byte(rng);
        } else if (mode == 2) {                // one header word set to an extreme value
            static const uint64_t ext[] = {0, 1, 0x7FFFFFFFull, 0x80000000ull, 0xFFFFFFFFull,
                                           0x7FFFFFFFFFFFFFFFull, 0x8000000000000000ull, ~0ull};
            const size_t w = (rng() % (512 / 8)) * 8;
            const uint64_t v = ext[rng() % 8];
            std::memcpy(img.data() + w, &v, (rng() & 1) ? 8 : 4);
        } else if (mode == 3) {                // truncation
            img.resize(rng() % img.size());
        } else if (mode == 4) {                // a region's offset or size moved (offsets at 104, sizes at 200)
            const size_t r = rng() % LW_REG_COUNT;
            const size_t at = ((rng() & 1) ? 104 : 200) + 8 * r;
            uint64_t v;
            std::memcpy(&v, img.data() + at, 8);
            const int64_t delta[] = {-256, -4, -1, 1, 4, 256, 1 << 20, -(1 << 20)};
            v += (uint64_t)delta[rng() % 8];
            std::memcpy(img.data() + at, &v, 8);
        } else {                               // bytes of the table / offsets / split regions
            uint64_t off;
            const int r = (int)(rng() % 3) == 0 ? LW_REG_TABLE : (rng() & 1) ? LW_REG_TILE_OFF : LW_REG_SPLIT;
            std::memcpy(&off, img.data() + 104 + 8 * r, 8);
            if (off < img.size()) img[off + rng() % std::min<size_t>(64, img.size() - off)] = (uint8_t)byte(rng);
        }
        exercise(img);
    }
}

int main(int argc, char **argv)
{
    const int iters = argc > 1 ? std::atoi(argv[1]) : 2000;
    const int64_t R = 128, C = 1280;
    std::vector<uint8_t> q4(R * C), q6(R * C);
    std::vector<uint16_t> d(R * C / 256), w(R * C);
    std::normal_distribution<double> nd(7.5, 1.8), nd6(31.5, 5.0), nw(0.0, 0.02);
    for (auto &v : q4) v = (uint8_t)std::min(15.0, std::max(0.0, std::nearbyint(nd(rng))));
    for (auto &v : q6) v = (uint8_t)std::min(63.0, std::max(0.0, std::nearbyint(nd6(rng))));
    for (auto &v : d) v = 0x2000 + (uint16_t)(rng() % 512);
    for (size_t i = 0; i < w.size(); i++) {
        float f = (float)nw(rng);
        if (rng() % 500 == 0) f *= 1e4f;       // outliers: verbatim segments
        uint32_t u;
        std::memcpy(&u, &f, 4);
        w[i] = (uint16_t)((u + 0x7FFF + ((u >> 16) & 1)) >> 16);
    }
    std::vector<std::vector<uint8_t>> images;
    lw_bundle *b = nullptr;
    CHECK(lw_bundle_build_q(LW_Q4_PAIR, R, C, q4.data(), d.data(), d.data(), &b) == LW_OK);
    images.push_back(image_of(b));
    lw_bundle_free(b);
    CHECK(lw_bundle_build_q_compact(LW_Q4_PAIR, R, C, q4.data(), d.data(), d.data(), &b) == LW_OK);
    images.push_back(image_of(b));
    lw_bundle_free(b);
    CHECK(lw_bundle_build_q(LW_Q6_SINGLE, R, C, q6.data(), d.data(), d.data(), &b) == LW_OK);
    images.push_back(image_of(b));
    lw_bundle_free(b);
    CHECK(lw_bundle_build_bf16(R, C, w.data(), &b) == LW_OK);
    images.push_back(image_of(b));
    lw_bundle_free(b);
    CHECK(lw_bundle_build_bf16_compact(R, C, w.data(), &b) == LW_OK);
    images.push_back(image_of(b));
    lw_bundle_free(b);

    // argument errors of the builders
    CHECK(lw_bundle_build_q(LW_Q4_PAIR, 65, C, q4.data(), d.data(), d.data(), &b) == LW_E_SHAPE);
    CHECK(lw_bundle_build_q(9, R, C, q4.data(), d.data(), d.data(), &b) == LW_E_ARG);
    CHECK(lw_bundle_build_q(LW_Q4_PAIR, R, C, nullptr, d.data(), d.data(), &b) == LW_E_ARG);
    CHECK(lw_bundle_build_q(LW_Q4_PAIR, R, C, q6.data(), d.data(), d.data(), &b) == LW_E_ARG);   // codes > 15
    CHECK(lw_bundle_build_q(LW_Q4_PAIR, -64, C, q4.data(), d.data(), d.data(), &b) == LW_E_SHAPE);
    std::vector<uint8_t> lens(256, 12);
    CHECK(lw_bundle_build_q_lens(LW_Q4_PAIR, R, C, q4.data(), d.data(), d.data(), lens.data(), &b) == LW_E_TABLE);
    std::fill(lens.begin(), lens.end(), 1);
    CHECK(lw_bundle_build_q_lens(LW_Q4_PAIR, R, C, q4.data(), d.data(), d.data(), lens.data(), &b) == LW_E_TABLE);
    CHECK(lw_bundle_load(nullptr, 10, &b) == LW_E_ARG);
    CHECK(lw_bundle_load(images[0].data(), 100, &b) == LW_E_FORMAT);

    for (const auto &img : images) fuzz_image(img, iters);
    std::printf("bundle_fuzz: %zu images x %d mutations, %d failed checks\n", images.size(), iters, fails);
    return fails ? 1 : 0;
}
