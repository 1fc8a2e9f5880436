// Host-side check of the decode work split's arithmetic (kvc_kernels.h): the
// slice table, the lookup of a key's slice, the small-quotient division and
// the exact division by H_kv. Prints one line per failure and exits non-zero.
#include "kvc_kernels.h"

#include <cstdio>
#include <cstdlib>
#include <random>

using kvc::DecodeArgs;

static int failures = 0;
#define CHECK(cond, ...)                      \
    do {                                      \
        if (!(cond)) {                        \
            if (++failures <= 20) {           \
                std::printf(__VA_ARGS__);     \
                std::printf("\n");            \
            }                                 \
        }                                     \
    } while (0)

// every slice is the previous one's end; every key lies in the slice that holds it
static void check_split(int64_t total, int n_cu, int per_cu, int64_t min_keys, int late, int odd) {
    DecodeArgs a{};
    a.total_keys = total;
    a.rows = 1;
    a.Hkv = 1;
    a.rec_rows = 4;
    a.ws_rows_cap = int64_t(1) << 40;
    kvc::decode_split_slices(a, n_cu, per_cu, min_keys, late, odd);
    CHECK(a.n_blocks >= 1 && a.n_blocks <= kvc::kMaxDecodeBlocks, "n_blocks %d", a.n_blocks);
    int64_t x = 0;
    for (int64_t k = 0; k < a.n_blocks; ++k) {
        const int64_t b = kvc::decode_slice_begin(a, k), n = kvc::decode_slice_size(a, k);
        CHECK(b == x, "total %lld: slice %lld begins at %lld, previous ended at %lld", (long long)total,
              (long long)k, (long long)b, (long long)x);
        CHECK(n >= 1, "slice %lld empty", (long long)k);
        CHECK(kvc::decode_slice_of(a, b) == k, "total %lld: slice_of(begin(%lld)) = %lld", (long long)total,
              (long long)k, (long long)kvc::decode_slice_of(a, b));
        const int64_t last = b + n - 1 < total - 1 ? b + n - 1 : total - 1;
        if (b < total)
            CHECK(kvc::decode_slice_of(a, last) == k, "total %lld: slice_of(%lld) = %lld, want %lld",
                  (long long)total, (long long)last, (long long)kvc::decode_slice_of(a, last), (long long)k);
        x = b + n;
    }
    CHECK(x >= total, "total %lld: slices end at %lld", (long long)total, (long long)x);
    CHECK(kvc::decode_slice_begin(a, a.n_blocks - 1) < total, "last slice past the axis");
}

int main() {
    std::mt19937_64 rng(7);
    // the launch shapes of the kernels: 256 CUs, 2, 3, 4 or 8 work-groups per CU, the
    // weights in use and around them, axes from a few keys to billions
    const int64_t totals[] = {1, 2, 31, 64, 65, 1000, 4097, 676736 + 256 * 48, 2097216 + 64 * 48,
                              (int64_t(1) << 31) + 12345, (int64_t(1) << 40) + 3};
    for (int64_t t : totals)
        for (int per_cu : {2, 3, 4, 8})
            for (int odd : {86, 88, 90, 100})
                for (int late : {70, 100}) check_split(t, 256, per_cu, 64, late, odd);
    for (int i = 0; i < 3000; ++i) {
        const int64_t t = 1 + static_cast<int64_t>(rng() % (int64_t(1) << (1 + rng() % 40)));
        check_split(t, 1 + static_cast<int>(rng() % 304), 1 + static_cast<int>(rng() % 8), 1 + rng() % 128,
                    50 + static_cast<int>(rng() % 51), 80 + static_cast<int>(rng() % 21));
    }
    // floor division with small quotients: exact at and around multiples
    for (int i = 0; i < 2000000; ++i) {
        const int64_t d = 1 + static_cast<int64_t>(rng() % (int64_t(1) << (1 + rng() % 45)));
        const int64_t qmax = (int64_t(1) << 31) - 1;
        int64_t q = static_cast<int64_t>(rng() % (1 + (rng() % 2 ? 1024 : qmax)));
        if (q > (int64_t(1) << 62) / d) q = (int64_t(1) << 62) / d;
        const int64_t r = static_cast<int64_t>(rng() % 3 == 0 ? (rng() % 2 ? 0 : d - 1) : rng() % d);
        const int64_t x = q * d + r;
        const int64_t got = kvc::decode_quot(x, d);
        CHECK(got == x / d, "decode_quot(%lld, %lld) = %lld, want %lld", (long long)x, (long long)d,
              (long long)got, (long long)(x / d));
    }
    // exact division by H_kv
    for (int h = 1; h <= 1024; ++h) {
        DecodeArgs a{};
        a.Hkv = h;
        kvc::decode_set_hkv_div(a);
        for (int i = 0; i < 2000; ++i) {
            const int64_t n = static_cast<int64_t>(rng() % (int64_t(1) << (1 + rng() % 40)));
            const int64_t got = kvc::decode_div_hkv(a, n * h);
            CHECK(got == n, "Hkv %d: %lld / Hkv = %lld, want %lld", h, (long long)(n * h), (long long)got,
                  (long long)n);
        }
    }
    std::printf("%s: %d failures\n", failures ? "FAIL" : "ok", failures);
    return failures ? 1 : 0;
}
