// Backward kernels of the Mamba-3 scan for bf16 inputs (m3_backward.hpp).
#include "m3_backward.hpp"

namespace m3 {
hipError_t launch_backward_bf16(const Dims& d, const BackwardArgs& a, const bwd::BwdWs& w, hipStream_t s) {
  return bwd::launch_io<bf16>(d, a, w, s);
}
}  // namespace m3
