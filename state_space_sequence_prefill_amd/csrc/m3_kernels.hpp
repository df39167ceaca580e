// Internal launch interface between the C ABI (m3_api.cpp) and the gfx950
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

struct Dims {
  int batch, heads, P, N, R, Q;
  bool bf16;
  int disc;  // m3_disc
};

// log2 of the rank padded to a power of two (the prefill tiles hold that
// many rows per token): 1 -> 0, 2 -> 1, 3..4 -> 2, 5..8 -> 3.
inline int pad_rank_log2(int R) { return R <= 1 ? 0 : R <= 2 ? 1 : R <= 4 ? 2 : 3; }

// Arguments of one decode step (see mamba3_decode_step in include/mamba3.h).
struct DecodeArgs {
  const void* x;
  const void* B;
  const void* C;
  const float* dt;
  const float* lam;
  const float* theta;
  const float* A;
  const float* D;
  float* h;
  void* B_prev;
  void* x_prev;
  void* y;
  int disc;  // m3_disc
  const void* gz;  // output epilogue, as in PrefillArgs
  const float* gw;
  float geps;
  const float* gdown;
  const float* nbw;  // BC normalisation, as in PrefillArgs
  const float* ncw;
  float neps;
};

// Arguments of the backward pass (mamba3_prefill_backward).
struct BackwardArgs {
  const void* x;
  const void* B;
  const void* C;
  const float* dt;
  const float* lam;
  const float* theta;
  const float* A;
  const float* D;
  const float* h;        // entry state of the prefill (lab frame)
  const void* B_prev;    // its pending pair
  const void* x_prev;
  const void* dy;        // cotangent of y (I/O dtype, y's layout)
  const float* dh_final; // cotangent of the final h, or nullptr
  float* dx;             // gradients, fp32, in the inputs' layouts
  float* dB;
  float* dC;
  float* ddt;
  float* dlam;
  float* dtheta;
  float* dA;             // (heads)
  float* dD;             // (heads)
  float* dh0;            // (batch, heads, P, N)
  float* dB_prev;        // (batch, heads, R, N)
  float* dx_prev;        // (batch, heads, R, P)
  void* ws;              // workspace (mamba3_prefill_backward_workspace_bytes)
  int seqlen;
  int disc;
};

// Arguments of one prefill pass over tokens [0, seqlen) of every chain.
struct PrefillArgs {
  const void* x;
  const void* B;
  const void* C;
  const float* dt;
  const float* lam;
  const float* theta;
  const float* A;
  const float* D;
  float* h;       // lab-frame state (batch, heads, P, N), in/out
  void* B_prev;   // pending B (batch, heads, R, N), in/out
  void* x_prev;   // pending x (batch, heads, R, P), in/out
  void* y;
  int disc;  // m3_disc
  // output epilogue (pre-gate grouped RMSNorm); gz == nullptr: plain y.
  // gdown != nullptr (with gz): MIMO rank down-projection (heads, R, P) first;
  // y and z are then (batch, T, heads, P)
  const void* gz;
  const float* gw;
  float geps;
  const float* gdown;
  // BC normalisation of the B and C rows before the scan (weights (heads, N)
  // each, applied to the pending B_prev as well, which stays raw in the
  // state); nbw == nullptr: none
  const float* nbw;
  const float* ncw;
  float neps;
  int seqlen;
  // Segment path (long prompts, few chains).  nseg == 1: plain fused pass.
  int nseg;        // number of segments the sequence is split into
  int seg_chunks;  // chunks per segment (the last segment may be shorter)
  float* seg_state;   // (nseg, batch, heads, P, N) fp32: per-segment summaries / start states
  float* seg_decay;   // (nseg, batch, heads) fp32: log of the segment's total decay
  float* seg_angle;   // (nseg, batch, heads, N/2) fp32: the segment's total angle
};

hipError_t launch_decode(const Dims& d, const DecodeArgs& a, hipStream_t s);
hipError_t launch_prefill(const Dims& d, const PrefillArgs& a, hipStream_t s);
// Zero three buffers, or copy three, in one launch (16-byte aligned pointers).
hipError_t launch_fill_zero3(void* const p[3], const size_t bytes[3], hipStream_t s);
hipError_t launch_copy3(void* const dst[3], const void* const src[3], const size_t bytes[3], hipStream_t s);

bool decode_supported(const Dims& d);
// Rank >= 2 decode on the matrix cores (m3_decode_mimo.hip).
bool decode_mimo_supported(const Dims& d);
hipError_t launch_decode_mimo(const Dims& d, const DecodeArgs& a, hipStream_t s);
bool prefill_supported(const Dims& d);

// Producer/consumer prefill (m3_prefill_pc.hip): used for every pass whose
// double-buffered tiles fit; `mode` 0 fused, 1 segment summaries, 2 segments.
bool prefill_pc_supported(const Dims& d);
// Whether the producer/consumer kernel serves these dims at some tile height:
// the gated epilogue and the BC normalisation live only there.
bool prefill_pc_path_supported(const Dims& d);
// Backward pass (m3_backward.hip).
bool backward_supported(const Dims& d);
size_t backward_workspace_bytes(const Dims& d, int seqlen);
hipError_t launch_backward(const Dims& d, const BackwardArgs& a, hipStream_t s);
// Chunk length the prefill kernels tile with (<= d.Q; see m3_prefill.hip).
int prefill_tile_chunk(const Dims& d);
hipError_t launch_prefill_pc(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks);
// The same with y stored through the output epilogue (m3_prefill_pc_gated.hip),
// and through the rank down-projection and the epilogue (m3_prefill_pc_down.hip).
hipError_t launch_prefill_pc_gated(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks);
hipError_t launch_prefill_pc_down(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks);
// The three variants with the BC normalisation in the producers' prep
// (m3_prefill_pc_bcnorm*.hip); epi 0 plain, 1 gated, 2 down-projected + gated.
hipError_t launch_prefill_pc_bcnorm(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks, int epi);
hipError_t launch_prefill_pc_bcnorm_gated(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks);
hipError_t launch_prefill_pc_bcnorm_down(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks);
// Whether the BC-normalisation instances serve these dims (their LDS holds
// the norm's weights and partial sums on top of the plain tiles).
bool prefill_pc_bcnorm_supported(const Dims& d);

// Device scratch of mamba3_prefill_noalloc (m3_noalloc.hip): a file-scope
// device array of kNoAllocScratchBytes per GPU; noalloc_scratch returns its
// device address on the current device (resolved once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace m3
