// Producer/consumer prefill (m3_prefill_pc.hpp) with the BC normalisation in
// the producers' prep (ai-flow-lab.com Mamba-3 summary, section
// "実装とカーネル最適化": BC/QK normalisation), plain y store; and the
// dispatch to the gated and down-projected variants, which compile in their
// own translation units.
#include "m3_prefill_pc.hpp"

namespace m3 {

hipError_t launch_prefill_pc_bcnorm(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks,
                                    int epi) {
  if (epi == kEpiGate) return launch_prefill_pc_bcnorm_gated(d, a, s, mode, nblocks);
  if (epi == kEpiDown) return launch_prefill_pc_bcnorm_down(d, a, s, mode, nblocks);
  return launch_pc<kEpiPlain, true>(d, a, s, mode, nblocks);
}

}  // namespace m3
