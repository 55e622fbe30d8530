// Kernel instantiations of the block-wise quantize / dequantize pair.
#include "launch.h"

namespace bitopt {

template <int DT, int BS>
static hipError_t quant_one(const CodecArgs& a, hipStream_t s) {
    constexpr int64_t tile = Layout<BS>::TE;
    hipLaunchKernelGGL((k_quantize<DT, BS>), tile_grid(a.n, tile), dim3(kThreads), 0, s, a);
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
