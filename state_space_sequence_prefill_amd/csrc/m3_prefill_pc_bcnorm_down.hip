// Producer/consumer prefill (m3_prefill_pc.hpp): BC normalisation in the
// prep, y through the MIMO rank down-projection and the output epilogue.
#include "m3_prefill_pc.hpp"

namespace m3 {

hipError_t launch_prefill_pc_bcnorm_down(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode,
                                         int nblocks) {
  return launch_pc<kEpiDown, true>(d, a, s, mode, nblocks);
}

}  // namespace m3
