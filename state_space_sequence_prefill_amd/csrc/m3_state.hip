// State initialisation and hand-off kernels (zero fill, device copy).
//
// The recurrent state is the fixed-size memory the pages contrast with a
// Transformer's growing KV cache (lilting.ch Mamba-3 article, section
// "SSMとは何か、Transformerの推論コスト問題"): an fp32 (P x N) matrix per
// (batch, head) plus the pending (B, x) of the last token.  Zeroing uses a
// fill kernel rather than hipMemsetAsync so that callers may capture it in a
// HIP graph.  Both kernels take a state's three buffers in one launch (a
// range of workgroups per buffer), move 16-byte vectors with a grid-stride
// loop and handle the byte tails.
#include "m3_device.hpp"
#include "m3_kernels.hpp"

namespace m3 {
namespace {

// Up to three buffers handled by one launch (a state's h, B_prev, x_prev):
// the grid's workgroups are split between them in proportion to their sizes
// (workgroups [b0[k], b0[k + 1]) take buffer k), each range walks its buffer
// grid-stride in 16-byte vectors, and its first workgroup writes the byte tail.
struct Bufs3 {
  uint4* d[3];
  const uint4* s[3];  // copy sources (unused by the fill)
  size_t n16[3];
  int ntail[3];
  unsigned b0[4];     // first workgroup of each buffer's range; b0[3] = grid size
};

__device__ __forceinline__ int which(const Bufs3& b) {
  const unsigned g = blockIdx.x;
  return g < b.b0[1] ? 0 : (g < b.b0[2] ? 1 : 2);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(Bufs3 b) {
  const int k = which(b);
  const size_t stride = (size_t)(b.b0[k + 1] - b.b0[k]) * blockDim.x;
  uint4* const d = b.d[k];
  const size_t n = b.n16[k];
  for (size_t i = (size_t)(blockIdx.x - b.b0[k]) * blockDim.x + threadIdx.x; i < n; i += stride)
    d[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == b.b0[k] && (int)threadIdx.x < b.ntail[k]) reinterpret_cast<uint8_t*>(d + n)[threadIdx.x] = 0;
}

// Copy: one vector per thread and iteration over many workgroups (measured
// on a 259 MiB state: up to 4096 workgroups this way moved 4.98 TB/s, four or
// eight loads in flight per thread over 256-2048 workgroups 4.2-4.9 TB/s).
__global__ __launch_bounds__(256) void copy_kernel(Bufs3 b) {
  const int k = which(b);
  const size_t stride = (size_t)(b.b0[k + 1] - b.b0[k]) * blockDim.x;
  uint4* const d = b.d[k];
  const uint4* const s = b.s[k];
  const size_t n = b.n16[k];
  for (size_t i = (size_t)(blockIdx.x - b.b0[k]) * blockDim.x + threadIdx.x; i < n; i += stride) d[i] = s[i];
  if (blockIdx.x == b.b0[k] && (int)threadIdx.x < b.ntail[k])
    reinterpret_cast<uint8_t*>(d + n)[threadIdx.x] = reinterpret_cast<const uint8_t*>(s + n)[threadIdx.x];
}

// Workgroups for a buffer of n16 vectors at `per_thread` vectors per thread
// (at least one, at most `cap`).
unsigned groups_for(size_t n16, int per_thread, unsigned cap) {
  size_t g = (n16 + 256 * (size_t)per_thread - 1) / (256 * (size_t)per_thread);
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

Bufs3 bufs3(void* const d[3], const void* const s[3], const size_t bytes[3], int per_thread) {
  Bufs3 b;
  b.b0[0] = 0;
  for (int k = 0; k < 3; ++k) {
    b.d[k] = static_cast<uint4*>(d[k]);
    b.s[k] = static_cast<const uint4*>(s ? s[k] : nullptr);
    b.n16[k] = bytes[k] / 16;
    b.ntail[k] = (int)(bytes[k] % 16);
    b.b0[k + 1] = b.b0[k] + groups_for(b.n16[k], per_thread, 4096);
  }
  return b;
}

}  // namespace

hipError_t launch_fill_zero3(void* const p[3], const size_t bytes[3], hipStream_t s) {
  if (bytes[0] + bytes[1] + bytes[2] == 0) return hipSuccess;
  const Bufs3 b = bufs3(p, nullptr, bytes, 1);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(b.b0[3]), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_copy3(void* const dst[3], const void* const src[3], const size_t bytes[3], hipStream_t s) {
  if (bytes[0] + bytes[1] + bytes[2] == 0) return hipSuccess;
  const Bufs3 b = bufs3(dst, src, bytes, 1);
  hipLaunchKernelGGL(copy_kernel, dim3(b.b0[3]), dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace m3
