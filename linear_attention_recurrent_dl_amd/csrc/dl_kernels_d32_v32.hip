// Decode / eager / merge kernel instantiations for d_k = d_v = 32, value tiles of 32 columns.
#include "dl_kernels.hpp"

namespace dl {
template hipError_t launch_step_d<32, 32>(int, int, int, int, int, const StepParams &, size_t, hipStream_t);
}  // namespace dl
