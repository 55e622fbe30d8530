// search_layout.h -- bucket layout of the nearest-code search tables.
//
// A bucket is addressed by a float's exponent and its top kM mantissa bits
// (v_bfe of bits 23-kM .. 30), clamped to the binades 2^-24 .. 2^1 (smaller
// magnitudes share the lowest bucket, larger ones and infinities the highest).
// Negative values use a mirrored half so that the bucket index is non-decreasing
// in x:  idx(x) = kNBH + (b ^ (sign ? ~0 : 0)),  b = clamp(key) - kKLO.
#pragma once

namespace bitopt {
namespace search {

constexpr int kM = 7;                                  // mantissa bits per binade
constexpr int kKLO = (127 - 24) << kM;                 // first key: binade 2^-24
constexpr int kKHI = (128 << kM) - 1;                  // last key: top of binade [1, 2)
constexpr int kNBH = kKHI - kKLO + 1;                  // buckets per sign
constexpr int kNB = 2 * kNBH;                          // buckets per map

}  // namespace search
}  // namespace bitopt
