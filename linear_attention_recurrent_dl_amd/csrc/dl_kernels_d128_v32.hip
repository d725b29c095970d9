// Decode / eager / merge / window kernel instantiations for d_k = d_v = 128, value tiles of 32 columns.
#include "dl_kernels.hpp"
#include "dl_window.hpp"

namespace dl {
template hipError_t launch_step_d<128, 32>(int, int, int, int, int, const StepParams &, size_t, hipStream_t);
template hipError_t launch_window_d<128, 32>(int, int, int, int, const WindowParams &, size_t, hipStream_t);
}  // namespace dl
