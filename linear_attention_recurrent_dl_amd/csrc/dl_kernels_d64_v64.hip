// Decode / eager / merge / window kernel instantiations for d_k = d_v = 64, value tiles of 64 columns.
#include "dl_kernels.hpp"
#include "dl_window.hpp"

namespace dl {
template hipError_t launch_step_d<64, 64>(int, int, int, int, int, const StepParams &, size_t, hipStream_t);
template hipError_t launch_window_d<64, 64>(int, int, int, int, const WindowParams &, size_t, hipStream_t);
}  // namespace dl
