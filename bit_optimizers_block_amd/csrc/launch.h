// launch.h -- internal interface between the C ABI (bitopt_api.cpp) and the
// translation units that instantiate the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace bitopt {

// Fused step (8-bit when quant, else fp32 states) for one optimizer family.
hipError_t launch_step_adam(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s);
hipError_t launch_step_ademamix(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s);
hipError_t launch_step_momentum(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s);
hipError_t launch_step_lion(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s);

hipError_t launch_quantize(const CodecArgs& a, int dtype, int bs, hipStream_t s);
hipError_t launch_dequantize(const CodecArgs& a, int dtype, int bs, hipStream_t s);

// Grid for a wave-per-tile kernel over n elements in tiles of `tile` elements.
inline dim3 tile_grid(int64_t n, int64_t tile) {
    const int64_t tiles = (n + tile - 1) / tile;
    int64_t groups = (tiles + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups > (1 << 22)) groups = 1 << 22;   // grid-stride beyond this
    if (groups < 1) groups = 1;
    return dim3((unsigned)groups);
}

template <int OPT>
hipError_t launch_step_family(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s);

}  // namespace bitopt
