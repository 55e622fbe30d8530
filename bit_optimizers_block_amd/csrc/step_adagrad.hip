// Kernel instantiations of the fused step for one optimizer family.
#include "step_dispatch.h"

namespace bitopt {
hipError_t launch_step_adagrad(const StepArgs& a, int dtype, int bs, bool quant, bool skip, bool unorm, hipStream_t s) {
    return launch_step_family<kAdagrad>(a, dtype, bs, quant, skip, unorm, s);
}
}  // namespace bitopt
