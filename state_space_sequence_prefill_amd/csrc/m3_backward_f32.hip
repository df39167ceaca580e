// Backward kernels of the Mamba-3 scan for fp32 inputs (m3_backward.hpp).
#include "m3_backward.hpp"

namespace m3 {
hipError_t launch_backward_f32(const Dims& d, const BackwardArgs& a, const bwd::BwdWs& w, hipStream_t s) {
  return bwd::launch_io<float>(d, a, w, s);
}
}  // namespace m3
