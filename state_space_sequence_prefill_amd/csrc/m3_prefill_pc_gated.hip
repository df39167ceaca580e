// Producer/consumer prefill (m3_prefill_pc.hpp) with y stored through the
// output epilogue (pre-gate grouped RMSNorm; ai-flow-lab.com Mamba-3 summary,
// section "実装とカーネル最適化").  A translation unit of its own so that the
// plain instances keep their register allocation and the two sets compile in
// parallel.
#include "m3_prefill_pc.hpp"

namespace m3 {

hipError_t launch_prefill_pc_gated(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks) {
  return launch_pc<kEpiGate, false>(d, a, s, mode, nblocks);
}

}  // namespace m3
