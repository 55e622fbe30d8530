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
hipError_t launch_step_rmsprop(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s);
hipError_t launch_step_adagrad(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s);

// Tensor-wide (non-block-wise) 8-bit step: clear, pass 1 (absmax), pass 2 (apply).
hipError_t launch_tensorwise(const StepArgs& a, int opt, int dtype, bool skip, hipStream_t s);
int tensorwise_workspace_words();
// The library's own tensor-wide workspace on the current device (a device array of
// tensorwise_scratch_words() words, shared by every call on that device).
hipError_t tensorwise_scratch(uint32_t** out);
int tensorwise_scratch_words();

hipError_t launch_quantize(const CodecArgs& a, int dtype, int bs, hipStream_t s);
hipError_t launch_dequantize(const CodecArgs& a, int dtype, int bs, hipStream_t s);

// Upper bound on the grid for the current device: compute units times the groups
// per CU the step kernels are launched with (CU count queried once per device).
// resident_per_cu > 0: that many groups per CU (a grid that is resident at once);
// 0: 256 per CU, i.e. one tile per wave for any tensor of practical size.  The
// environment variable BITOPT_GROUPS_PER_CU overrides both.
int64_t group_cap(int resident_per_cu = 0);

// Groups of `kernel` (kThreads threads, static LDS only) resident on one CU.
int resident_groups_per_cu(const void* kernel);

// Grid for a wave-per-tile kernel over n elements in tiles of `tile` elements:
// one tile per wave up to group_cap() groups, grid-stride beyond.
inline dim3 tile_grid(int64_t n, int64_t tile, int resident_per_cu = 0) {
    const int64_t tiles = (n + tile - 1) / tile;
    int64_t groups = (tiles + kWavesPerGroup - 1) / kWavesPerGroup;
    const int64_t cap = group_cap(resident_per_cu);
    if (groups > cap) groups = cap;
    if (groups < 1) groups = 1;
    return dim3((unsigned)groups);
}

template <int OPT>
hipError_t launch_step_family(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s);

}  // namespace bitopt
