// Kernel instantiations of the block-wise quantize / dequantize pair.
#include "launch.h"

namespace bitopt {

// quantize runs a resident grid -- as many groups per CU as its occupancy allows, each
// wave looping over tiles -- so that each group stages the map and its search tables
// (about 10 KB) once rather than once per four tiles: 4096x4096 fp32 0.653 -> 0.673 of
// HBM peak, bf16 0.505 -> 0.588 (one box).  dequantize stages 1 KB and keeps one tile per
// wave (a resident grid measured slower).
template <int DT, int BS>
static hipError_t quant_one(const CodecArgs& a, hipStream_t s) {
    constexpr int64_t tile = Layout<BS>::TE;
    static const int per_cu = resident_groups_per_cu(reinterpret_cast<const void*>(&k_quantize<DT, BS>));
    hipLaunchKernelGGL((k_quantize<DT, BS>), tile_grid(a.n, tile, per_cu), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int DT, int BS>
static hipError_t dequant_one(const CodecArgs& a, hipStream_t s) {
    constexpr int64_t tile = Layout<BS>::TE;
    hipLaunchKernelGGL((k_dequantize<DT, BS>), tile_grid(a.n, tile), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t quant_bs(const CodecArgs& a, int bs, hipStream_t s) {
    if (bs == 256) return quant_one<DT, 256>(a, s);
    if (bs == 2048) return quant_one<DT, 2048>(a, s);
    return hipErrorInvalidValue;
}

template <int DT>
static hipError_t dequant_bs(const CodecArgs& a, int bs, hipStream_t s) {
    if (bs == 256) return dequant_one<DT, 256>(a, s);
    if (bs == 2048) return dequant_one<DT, 2048>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_quantize(const CodecArgs& a, int dtype, int bs, hipStream_t s) {
    switch (dtype) {
    case kF32: return quant_bs<kF32>(a, bs, s);
    case kF16: return quant_bs<kF16>(a, bs, s);
    case kBF16: return quant_bs<kBF16>(a, bs, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dequantize(const CodecArgs& a, int dtype, int bs, hipStream_t s) {
    switch (dtype) {
    case kF32: return dequant_bs<kF32>(a, bs, s);
    case kF16: return dequant_bs<kF16>(a, bs, s);
    case kBF16: return dequant_bs<kBF16>(a, bs, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bitopt
