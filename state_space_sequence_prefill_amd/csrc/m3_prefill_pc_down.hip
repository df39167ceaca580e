// Producer/consumer prefill (m3_prefill_pc.hpp) with the MIMO rank
// down-projection folded into the output tile (lilting.ch Mamba-3 article,
// "3. MIMO SSM": the rank-r output returns to the P channels) and the output
// epilogue after it (pre-gate grouped RMSNorm; ai-flow-lab.com Mamba-3
// summary, section "実装とカーネル最適化").  y and z are (batch, T, heads, P).
#include "m3_prefill_pc.hpp"

namespace m3 {

hipError_t launch_prefill_pc_down(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks) {
  return launch_pc<kEpiDown, false>(d, a, s, mode, nblocks);
}

}  // namespace m3
