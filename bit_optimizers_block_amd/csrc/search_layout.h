// search_layout.h -- bucket layout of the nearest-code search tables.
//
// The table encoder is handed y' = y * 2^-kShift, where y is the normalized state
// value (|y| < 2 for finite data: |s| <= A' and fl(1/A') * A' <= 1 + 2^-23).  A
// bucket is addressed by bits 16 .. 27 of y': the low 5 bits of its exponent and its
// top kM mantissa bits.  For |y| in [2^-30, 2) the exponent field of y' is 1 .. 31,
// so those 12 bits name the binade and the sub-binade exactly; smaller magnitudes
// have exponent field 0 (keys 0 .. 127, all of them below the first threshold), and
// infinities and NaN alias into the top binade, so the key is always in range and
// needs no clamp.  Finite blocks stay below 1 + 2^-7 there (key 0xF80); keys 0xF81 ..
// 0xFFF are reached only by (quiet) NaN, and their buckets hold the code of +0.  Negative values use a mirrored half, which keeps the bucket index
// non-decreasing in y:  idx(y) = kNBH + (key ^ (sign ? ~0 : 0)).  Values known to be
// non-negative skip the sign term: idx = kNBH + key.
#pragma once

namespace bitopt {
namespace search {

constexpr int kM = 7;                                  // mantissa bits per binade
constexpr int kShift = 96;                             // y' = y * 2^-kShift
constexpr int kKeyBits = 5 + kM;                       // low exponent bits + mantissa bits
constexpr int kNBH = 1 << kKeyBits;                    // buckets per sign
constexpr int kNB = 2 * kNBH;                          // buckets per map
// The scaled value is exact (y' = y * 2^-kShift with one rounding) when the block's
// reciprocal r satisfies r * 2^-kShift >= 2^-126, i.e. r >= 2^(kShift - 126).
constexpr int kMinRecipExp = kShift - 126;

}  // namespace search
}  // namespace bitopt
