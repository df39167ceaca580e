// Host-only stand-ins for the kernel side of the scan library, so that the C
// ABI's validation layer (m3_api.cpp) can be built with AddressSanitizer and
// UndefinedBehaviorSanitizer by a host compiler and driven without a GPU.
// Size predicates follow the library's supported set in outline (the real
// ones live beside the kernels); every launch returns hipErrorNoDevice, which
// the ABI reports as M3_ERR_HIP.  Test infrastructure only.
#include "../../state_space_sequence_prefill_amd/csrc/m3_kernels.hpp"

namespace m3 {
namespace {
bool p_ok(int P) { return P == 16 || P == 32 || P == 64 || P == 128; }
bool n_ok(int N) { return N == 16 || N == 32 || N == 64 || N == 128 || N == 256; }
}  // namespace

bool prefill_supported(const Dims& d) {
  return p_ok(d.P) && n_ok(d.N) && d.R >= 1 && d.R <= 8 && (d.Q == 16 || d.Q == 32 || d.Q == 64);
}
bool decode_supported(const Dims& d) { return p_ok(d.P) && n_ok(d.N) && d.R >= 1 && d.R <= 8; }
bool decode_mimo_supported(const Dims& d) { return decode_supported(d) && d.R >= 2; }
bool prefill_pc_supported(const Dims& d) { return prefill_supported(d); }
bool prefill_pc_path_supported(const Dims& d) { return prefill_supported(d); }
bool prefill_pc_bcnorm_supported(const Dims& d) { return prefill_supported(d); }
int prefill_tile_chunk(const Dims& d) { return d.Q; }
bool backward_supported(const Dims& d) {
  return (d.R == 1 || d.R == 2 || d.R == 4) && d.P % 16 == 0 && d.N % 16 == 0 && d.P <= 128 && d.N <= 128;
}
size_t backward_workspace_bytes(const Dims& d, int seqlen) {
  return (size_t)d.batch * d.heads * (size_t)(seqlen + 1) * d.P * d.N * 4;
}
hipError_t launch_decode(const Dims&, const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(const Dims&, const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fill_zero3(void* const*, const size_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_copy3(void* const*, const void* const*, const size_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_backward(const Dims&, const BackwardArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch(void**) { return hipErrorNoDevice; }

}  // namespace m3
