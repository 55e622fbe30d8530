// Kernel instantiations and launches of the tensor-wide (non-block-wise) 8-bit step.
#include <mutex>

#include "launch.h"
#include "tensorwise.h"

namespace bitopt {

// Workspace of the allocation-free tensor-wide step: a file-scope device array, one
// copy per GPU, held until the process ends.  In host code `scratch` only names the
// symbol; its device address is looked up once per device (tensorwise_scratch) and
// only that address is handed to kernels.
static __device__ __align__(256) uint32_t scratch[kTwWords];

hipError_t tensorwise_scratch(uint32_t** out) {
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void* ptrs[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptrs[dev] = p;
    }
    *out = static_cast<uint32_t*>(ptrs[dev]);
    return hipSuccess;
}

int tensorwise_scratch_words() { return kTwWords; }

namespace {

template <int DT, int OPT, bool SKIP, bool UNORM>
hipError_t tw_launch(const StepArgs& a0, hipStream_t s) {
    StepArgs a = a0;
    const dim3 grid = tile_grid(a.n, 1024);
    const int64_t tiles = (a.n + 1023) / 1024;
    int64_t parts = (tiles + kWavesPerGroup - 1) / kWavesPerGroup;
    if (parts > kTwMaxParts) parts = kTwMaxParts;
    a.parts = (int32_t)parts;
    hipLaunchKernelGGL((k_tw_max<DT, OPT, SKIP, UNORM>), dim3((unsigned)parts), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL((k_tw_reduce<OPT, UNORM>), dim3(1), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL((k_tw_apply<DT, OPT, SKIP, UNORM>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int DT, int OPT>
hipError_t tw_skip(const StepArgs& a, bool skip, hipStream_t s) {
    const bool unorm = a.s.max_unorm > 0.0f;
    if (skip) return unorm ? tw_launch<DT, OPT, true, true>(a, s) : tw_launch<DT, OPT, true, false>(a, s);
    return unorm ? tw_launch<DT, OPT, false, true>(a, s) : tw_launch<DT, OPT, false, false>(a, s);
}

template <int OPT>
hipError_t tw_dtype(const StepArgs& a, int dtype, bool skip, hipStream_t s) {
    switch (dtype) {
    case kF32: return tw_skip<kF32, OPT>(a, skip, s);
    case kF16: return tw_skip<kF16, OPT>(a, skip, s);
    case kBF16: return tw_skip<kBF16, OPT>(a, skip, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int tensorwise_workspace_words() { return kTwWords; }

hipError_t launch_tensorwise(const StepArgs& a, int opt, int dtype, bool skip, hipStream_t s) {
    switch (opt) {
    case kAdam: return tw_dtype<kAdam>(a, dtype, skip, s);
    case kAdemamix: return tw_dtype<kAdemamix>(a, dtype, skip, s);
    case kMomentum: return tw_dtype<kMomentum>(a, dtype, skip, s);
    case kLion: return tw_dtype<kLion>(a, dtype, skip, s);
    case kRmsprop: return tw_dtype<kRmsprop>(a, dtype, skip, s);
    case kAdagrad: return tw_dtype<kAdagrad>(a, dtype, skip, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bitopt
