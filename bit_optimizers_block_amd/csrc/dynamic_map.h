// dynamic_map.h -- host construction of the dynamic-exponent codebooks
// ("8-bit Optimizers via Block-wise Quantization": abstract, and the quote on
// dynamic exponent data types among its citing papers: a sign bit, then a run of
// zero bits selecting a base-10 exponent, then fraction bits).
#pragma once

#include <algorithm>
#include <cmath>

namespace bitopt {

// Signed map: for each decade 10^-E (E = 0..6), the 2^(6-E) midpoints of equal
// bins of [0.1, 1] * 10^-E, with both signs.  Unsigned map: 2^(7-E) midpoints per
// decade (the sign bit becomes a fraction bit).  Both add exact 0 and +1.0.
// Values are formed in double, rounded once to fp32 and sorted ascending.
inline void build_dynamic_map(bool is_signed, float out[256]) {
    const int top_bits = is_signed ? 6 : 7;
    int k = 0;
    out[k++] = 0.0f;
    out[k++] = 1.0f;
    for (int E = 0; E <= 6; ++E) {
        const int bits = top_bits - E;
        const double bins = (double)(1 << bits);
        const double scale = std::pow(10.0, -(double)E);
        for (int f = 0; f < (1 << bits); ++f) {
            const double mid = 0.1 + 0.9 * ((double)f + 0.5) / bins;
            const float v = (float)(scale * mid);
            out[k++] = v;
            if (is_signed) out[k++] = -v;
        }
    }
    std::sort(out, out + 256);
}

}  // namespace bitopt
