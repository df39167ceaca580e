// Producer/consumer prefill (m3_prefill_pc.hpp): the instances that store the
// plain scan output, the support test, and the dispatch between the plain
// and the gated instances.
#include "m3_prefill_pc.hpp"

namespace m3 {

bool prefill_pc_supported(const Dims& d) {
  const int rows_pad = ((d.Q << pad_rank_log2(d.R)) + 31) & ~31;
  return rows_pad <= (d.bf16 ? pc_max_rows<bf16>(d) : pc_max_rows<float>(d));
}

bool prefill_pc_bcnorm_supported(const Dims& d) {
  return prefill_pc_path_supported(d) && (d.bf16 ? pc_bcn_fits<bf16>(d) : pc_bcn_fits<float>(d));
}

hipError_t launch_prefill_pc(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks) {
  // segment summaries write no y, so they never need the epilogue
  const int epi = (a.gz && mode != kPcSummary) ? (a.gdown ? kEpiDown : kEpiGate) : kEpiPlain;
  if (a.nbw) return launch_prefill_pc_bcnorm(d, a, s, mode, nblocks, epi);
  if (epi == kEpiGate) return launch_prefill_pc_gated(d, a, s, mode, nblocks);
  if (epi == kEpiDown) return launch_prefill_pc_down(d, a, s, mode, nblocks);
  return launch_pc<kEpiPlain, false>(d, a, s, mode, nblocks);
}

}  // namespace m3
