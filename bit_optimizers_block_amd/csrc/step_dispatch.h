// step_dispatch.h -- maps the run-time (dtype, blocksize, mode, flags) of a step
// call to its kernel instantiation.  Included once per optimizer family, so each
// family's kernels compile in their own translation unit.
#pragma once

#include "launch.h"

namespace bitopt {

// Grid policy.  Single-tensor 8-bit steps of the root optimizers (Adam, AdEMAMix,
// RMSprop, Adagrad) on 16-bit parameters -- the most arithmetic per byte -- run a
// resident grid: as many groups per CU as fit at once, each wave looping over
// tiles, so the codebooks and search tables are staged once per group rather than
// once per four tiles (+2..7% over one tile per wave, A/B on one GPU).  Multi-tensor
// launches use 512 groups per CU (a grid stride of a few tiles per wave).
// Everything else keeps one tile per wave, which measured faster: fp32 parameters,
// Momentum and Lion (fewer instructions per byte: -6..9% with a resident grid), and
// skip_zeros launches, whose all-zero groups end early only when the grid covers
// every tile.
template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM, bool MULTI>
int grid_groups_per_cu() {
    if constexpr (MULTI) {
        // Multi-tensor launches (hundreds of millions of elements): 512 groups per CU,
        // i.e. about two and a half tiles per wave for the 1.3 G-parameter set, ran 1%
        // faster than 256 and 3-5% faster than 1024 or 4096 (one GPU, bf16 Adam).
        return 512;
    } else if constexpr (DT == kF32 || !QUANT || SKIP || !HasRoot<OPT>::v) {
        return 0;
    } else {
        static const int n =
            resident_groups_per_cu(reinterpret_cast<const void*>(&k_step<DT, OPT, BS, QUANT, SKIP, UNORM, MULTI>));
        return n;
    }
}

template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM>
hipError_t launch_one(const StepArgs& a, hipStream_t s) {
    constexpr int64_t tile = Layout<BS>::TE;
    if constexpr (PairBlocks<BS, QUANT, SKIP, UNORM, false>::v) {
        if (!a.table) {
            // wave pairs: two 2048-element blocks per group and iteration
            int64_t groups = (a.nb + 1) / 2;
            const int64_t cap = group_cap(grid_groups_per_cu<DT, OPT, BS, QUANT, SKIP, UNORM, false>());
            if (groups > cap) groups = cap;
            if (groups < 1) groups = 1;
            hipLaunchKernelGGL((k_step<DT, OPT, BS, QUANT, SKIP, UNORM, false>), dim3((unsigned)groups),
                               dim3(kThreads), 0, s, a);
            return hipGetLastError();
        }
    }
    if (a.table)
        hipLaunchKernelGGL((k_step<DT, OPT, BS, QUANT, SKIP, UNORM, true>),
                           tile_grid(a.total_tiles * tile, tile, grid_groups_per_cu<DT, OPT, BS, QUANT, SKIP, UNORM, true>()),
                           dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_step<DT, OPT, BS, QUANT, SKIP, UNORM, false>),
                           tile_grid(a.n, tile, grid_groups_per_cu<DT, OPT, BS, QUANT, SKIP, UNORM, false>()),
                           dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int DT, int OPT, int BS, bool QUANT>
hipError_t launch_flags(const StepArgs& a, bool skip, bool unorm, hipStream_t s) {
    if (skip) return unorm ? launch_one<DT, OPT, BS, QUANT, true, true>(a, s) : launch_one<DT, OPT, BS, QUANT, true, false>(a, s);
    return unorm ? launch_one<DT, OPT, BS, QUANT, false, true>(a, s) : launch_one<DT, OPT, BS, QUANT, false, false>(a, s);
}

template <int DT, int OPT>
hipError_t launch_bs(const StepArgs& a, int bs, bool quant, bool skip, bool unorm, hipStream_t s) {
    if (bs == 256) return quant ? launch_flags<DT, OPT, 256, true>(a, skip, unorm, s) : launch_flags<DT, OPT, 256, false>(a, skip, unorm, s);
    if (bs == 2048) return quant ? launch_flags<DT, OPT, 2048, true>(a, skip, unorm, s) : launch_flags<DT, OPT, 2048, false>(a, skip, unorm, s);
    return hipErrorInvalidValue;
}

template <int OPT>
hipError_t launch_step_family(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s) {
    switch (dtype) {
    case kF32: return launch_bs<kF32, OPT>(a, bs, quant, skip, unorm, s);
    case kF16: return launch_bs<kF16, OPT>(a, bs, quant, skip, unorm, s);
    case kBF16: return launch_bs<kBF16, OPT>(a, bs, quant, skip, unorm, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bitopt
