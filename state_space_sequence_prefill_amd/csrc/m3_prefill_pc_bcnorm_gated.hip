// Producer/consumer prefill (m3_prefill_pc.hpp): BC normalisation in the
// prep, y through the output epilogue (pre-gate grouped RMSNorm).
#include "m3_prefill_pc.hpp"

namespace m3 {

hipError_t launch_prefill_pc_bcnorm_gated(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode,
                                          int nblocks) {
  return launch_pc<kEpiGate, true>(d, a, s, mode, nblocks);
}

}  // namespace m3
