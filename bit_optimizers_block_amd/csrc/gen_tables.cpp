// gen_tables.cpp -- build-time generator of the constant code-search tables for
// the two standard dynamic maps.  Writes a header included by the kernels.
//
// Nearest code.  For a sorted map Q the nearest entry to x (fp32 distance, ties to
// the lower index) is a non-decreasing step function of x.  Its steps are the
// decision thresholds tau[j] = the smallest fp32 x at which the code exceeds j;
// tau[j] lies in (Q[j], Q[j+1]] and is found here by bisection over the ordered
// fp32 values, evaluating exactly the fp32 comparison the definition makes:
// (Q[j+1] - x) < (x - Q[j]).  Then code(x) = #{j : tau[j] <= x}.
//
// Bucket table.  The device looks values up scaled by 2^-kShift (search_layout.h):
// the fp32 line of y' = x * 2^-kShift is cut into buckets by the low 5 exponent bits
// and the top kM mantissa bits, each sign, and each bucket stores the code at its
// lower end.  The thresholds are stored scaled the same way (exact: every |tau| is
// far above 2^-30).  The generator checks that no bucket holds more than one
// threshold, so on the device
//     code(x) = bucket[idx(y')] + (y' >= tau'[bucket[idx(y')]]),
// and then replays that formula against a brute-force nearest-entry scan on values
// around every threshold and map entry and on random values; any difference fails
// the build.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <random>

#include "dynamic_map.h"
#include "search_layout.h"

namespace {

uint32_t f2u(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
float u2f(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

// Order-preserving key of a non-NaN float (-0 sorts just below +0).
uint32_t okey(float f) { const uint32_t u = f2u(f); return (u & 0x80000000u) ? ~u : (u | 0x80000000u); }
float unkey(uint32_t k) { return u2f((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }

bool upper_wins(const float* Q, int j, float x) {
    const float du = Q[j + 1] - x;
    const float dd = x - Q[j];
    return du < dd;
}

void thresholds(const float* Q, float tau[256]) {
    for (int j = 0; j < 255; ++j) {
        uint32_t lo = okey(Q[j]), hi = okey(Q[j + 1]);   // upper_wins: false at lo, true at hi
        if (upper_wins(Q, j, Q[j]) || !upper_wins(Q, j, Q[j + 1])) {
            std::fprintf(stderr, "gen_tables: non-monotone decision at %d\n", j);
            std::exit(1);
        }
        while (hi - lo > 1) {
            const uint32_t mid = lo + (hi - lo) / 2;
            if (upper_wins(Q, j, unkey(mid))) hi = mid; else lo = mid;
        }
        tau[j] = unkey(hi);
    }
    tau[255] = u2f(0x7fc00000u);   // NaN: "x >= tau[255]" is always false
}

int code_at(const float* tau, float x) {
    int c = 0;
    while (c < 255 && tau[c] <= x) ++c;
    return c;
}

// Value range [vmin, vmax] (scaled, y' space) of bucket index k.
void bucket_range(int k, float* vmin, float* vmax) {
    using namespace bitopt::search;
    const bool neg = k < kNBH;
    const uint32_t key = (uint32_t)(neg ? (kNBH - 1 - k) : (k - kNBH));
    const uint32_t mag_lo = key << 16;
    const uint32_t mag_hi = ((key + 1) << 16) - 1;
    if (!neg) { *vmin = u2f(mag_lo); *vmax = u2f(mag_hi); }
    else { *vmin = -u2f(mag_hi); *vmax = -u2f(mag_lo); }
}

// The device encoder on a scaled value: bucket, then one threshold comparison.
int table_code(const uint8_t* table, const float* tau_s, float ys, bool nonneg) {
    using namespace bitopt::search;
    const uint32_t bits = f2u(ys);
    const uint32_t key = (bits >> 16) & (uint32_t)(kNBH - 1);
    const uint32_t sgn = nonneg ? 0u : (uint32_t)((int32_t)bits >> 31);
    const uint32_t idx = (uint32_t)kNBH + (key ^ sgn);
    const int c = table[idx];
    return c + (ys >= tau_s[c] ? 1 : 0);
}

int brute_nearest(const float* Q, float x) {
    int best = 0;
    float bd = std::fabs(x - Q[0]);
    for (int j = 1; j < 256; ++j) {
        const float d = std::fabs(x - Q[j]);
        if (d < bd) { bd = d; best = j; }
    }
    return best;
}

// x * 2^-kShift rounded once to fp32, as the device's multiply by the scaled
// reciprocal gives it (exact for |x| >= 2^-30).
float scaled(float x) { return (float)std::ldexp((double)x, -bitopt::search::kShift); }

// Replay the table encoder against the brute-force scan; returns the mismatch count.
long verify(const float* Q, const float* tau, const uint8_t* table, const float* tau_s, bool is_signed) {
    long bad = 0, tested = 0;
    auto check = [&](float x) {
        if (!(std::fabs(x) <= 1.0000002f)) return;
        if (!is_signed && x < 0.0f) return;
        const int want = brute_nearest(Q, x);
        for (int nn = 0; nn < (x >= 0.0f && !std::signbit(x) ? 2 : 1); ++nn) {
            const int got = table_code(table, tau_s, scaled(x), nn == 1);
            ++tested;
            if (got != want) {
                if (bad < 10) std::fprintf(stderr, "gen_tables: x=%a nonneg=%d table %d nearest %d\n", x, nn, got, want);
                ++bad;
            }
        }
    };
    for (int j = 0; j < 256; ++j) {
        const float pts[2] = {Q[j], j < 255 ? tau[j] : Q[j]};
        for (float c : pts)
            for (int d = -64; d <= 64; ++d) {
                const uint32_t u = f2u(c);
                check(u2f(u + (uint32_t)d));
                check(-u2f(u + (uint32_t)d));
            }
    }
    std::mt19937 rng(12345);
    std::uniform_real_distribution<float> uni(-1.0f, 1.0f);
    std::uniform_real_distribution<float> lg(-40.0f, 0.0f);
    for (int i = 0; i < 200000; ++i) {
        check(uni(rng));
        const float m = (float)std::exp2((double)lg(rng));
        check(m);
        check(-m);
    }
    const float special[] = {0.0f, -0.0f, 1.0f, -1.0f, 0x1p-30f, 0x1p-31f, 0x1p-126f, 0x1p-149f, 1.0000001f};
    for (float x : special) check(x);
    // NaN (any sign, any quiet payload) encodes as +0 does
    const int want_nan = brute_nearest(Q, 0.0f);
    const uint32_t nans[] = {0x7fc00000u, 0xffc00000u, 0x7fc00001u, 0x7fffffffu, 0xffffffffu, 0xffd00000u};
    for (uint32_t u : nans)
        for (int nn = 0; nn < 2; ++nn) {
            ++tested;
            if (table_code(table, tau_s, u2f(u), nn == 1) != want_nan) {
                std::fprintf(stderr, "gen_tables: NaN %08x nonneg=%d does not encode as +0\n", u, nn);
                ++bad;
            }
        }
    if (tested == 0) return 1;
    return bad;
}

void emit_floats(FILE* f, const char* name, const float* v, int n) {
    std::fprintf(f, "alignas(16) static __device__ const uint32_t %s[%d] = {", name, n);
    for (int i = 0; i < n; ++i) std::fprintf(f, "%s0x%08xu", i % 8 ? ", " : ",\n    " + (i == 0), f2u(v[i]));
    std::fprintf(f, "};\n");
}

}  // namespace

int main(int argc, char** argv) {
    using namespace bitopt::search;
    if (argc != 2) { std::fprintf(stderr, "usage: gen_tables OUT.h\n"); return 2; }
    FILE* f = std::fopen(argv[1], "w");
    if (!f) { std::perror(argv[1]); return 1; }
    std::fprintf(f, "// Generated by gen_tables.cpp -- constant code-search tables of the standard\n"
                    "// dynamic maps (index 0: signed, 1: unsigned).  Do not edit.\n#pragma once\n#include <stdint.h>\n\n");
    for (int s = 0; s < 2; ++s) {
        float Q[256], tau[256];
        bitopt::build_dynamic_map(s == 0, Q);
        thresholds(Q, tau);
        float tau_s[256];
        for (int j = 0; j < 256; ++j) tau_s[j] = j < 255 ? (float)std::ldexp((double)tau[j], -kShift) : tau[j];
        for (int j = 0; j < 255; ++j)
            if (std::ldexp((double)tau_s[j], kShift) != (double)tau[j] || std::fabs(tau[j]) < 0x1p-30f) {
                std::fprintf(stderr, "gen_tables: threshold %d of map %d does not scale exactly\n", j, s);
                return 1;
            }
        static uint8_t table[kNB];
        for (int k = 0; k < kNB; ++k) {
            float vmin, vmax;
            bucket_range(k, &vmin, &vmax);
            const int c0 = code_at(tau_s, vmin), c1 = code_at(tau_s, vmax);
            if (c1 - c0 > 1) {
                std::fprintf(stderr, "gen_tables: bucket %d of map %d holds %d thresholds\n", k, s, c1 - c0);
                return 1;
            }
            table[k] = (uint8_t)c0;
        }
        // Keys above the top finite key (normalized magnitudes in [1 + 2^-7, 2), which
        // no finite block reaches: |y| <= 1 + 2^-23) are reached only by NaN, whose
        // exponent field is all ones and whose quiet bit sets the top mantissa bit.
        // They get the code of +0 (the encoding of a NaN value), and the threshold
        // comparison that follows is false for NaN.
        const int zero_code = brute_nearest(Q, 0.0f);
        for (int key = kNBH - (1 << kM) + 1; key < kNBH; ++key) {
            table[kNBH + key] = (uint8_t)zero_code;
            table[kNBH - 1 - key] = (uint8_t)zero_code;
        }
        const long bad = verify(Q, tau, table, tau_s, s == 0);
        if (bad) {
            std::fprintf(stderr, "gen_tables: table encoder disagrees with the nearest entry on %ld values (map %d)\n", bad, s);
            return 1;
        }
        char name[64];
        std::snprintf(name, sizeof name, "kStdQ%d", s);
        emit_floats(f, name, Q, 256);
        std::snprintf(name, sizeof name, "kStdTau%d", s);
        emit_floats(f, name, tau_s, 256);
        std::fprintf(f, "alignas(16) static __device__ const uint8_t kStdBucket%d[%d] = {", s, kNB);
        for (int k = 0; k < kNB; ++k) std::fprintf(f, "%s%u", k % 24 ? "," : ",\n    " + (k == 0), table[k]);
        std::fprintf(f, "};\n\n");
    }
    std::fclose(f);
    return 0;
}
