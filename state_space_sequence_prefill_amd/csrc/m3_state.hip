// State initialisation and hand-off kernels (zero fill, device copy).
//
// The recurrent state is the fixed-size memory the pages contrast with a
// Transformer's growing KV cache (lilting.ch Mamba-3 article, section
// "SSMとは何か、Transformerの推論コスト問題"): an fp32 (P x N) matrix per
// (batch, head) plus the pending (B, x) of the last token.  Zeroing uses a
// fill kernel rather than hipMemsetAsync so that callers may capture it in a
// HIP graph.  Both kernels move 16-byte vectors with a grid-stride loop and
// handle a byte tail.
#include "m3_device.hpp"
#include "m3_kernels.hpp"

namespace m3 {
namespace {

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16, uint8_t* tail, int ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void copy_kernel(uint4* __restrict__ d, const uint4* __restrict__ s,
                                                   size_t n16, uint8_t* dt, const uint8_t* st, int ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) d[i] = s[i];
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) dt[threadIdx.x] = st[threadIdx.x];
}

unsigned grid_for(size_t n16) {
  size_t g = (n16 + 255) / 256;
  if (g < 1) g = 1;
  if (g > 4096) g = 4096;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes % 16);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n16)), dim3(256), 0, s, static_cast<uint4*>(p), n16,
                     static_cast<uint8_t*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes % 16);
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n16)), dim3(256), 0, s, static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), n16, static_cast<uint8_t*>(dst) + n16 * 16,
                     static_cast<const uint8_t*>(src) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace m3
