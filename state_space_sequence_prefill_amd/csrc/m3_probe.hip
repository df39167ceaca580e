// Bandwidth probes for the measurement harness (libm3probe.so, not part of
// the scan library's ABI): how fast this GPU streams HBM when a kernel does
// nothing else, as the achievable ceiling beside the 8 TB/s specification.
//
//   read   every thread sums its 16-byte vectors (UNROLL loads in flight per
//          thread, grid-stride over the buffer); one float per workgroup out
//   write  every thread stores 16-byte vectors
//   copy   16-byte loads and stores
//
// Exported with C linkage: m3probe_read / m3probe_write / m3probe_copy
// (device pointers, byte counts that are multiples of 16, a workgroup count,
// a hipStream_t as void*), returning the hipError_t of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void probe_read(const uint4* __restrict__ src, size_t n16,
                                                       float* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = __uint_as_float(red[0] & 0x7fffffu);
}

__global__ __launch_bounds__(kThreads) void probe_write(uint4* __restrict__ dst, size_t n16, uint32_t v) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
    dst[i] = make_uint4(v, v, v, v);
}

__global__ __launch_bounds__(kThreads) void probe_copy(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                       size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

int m3probe_read(const void* src, size_t bytes, float* out, int blocks, void* stream) {
  hipLaunchKernelGGL(probe_read, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, out);
  return (int)hipGetLastError();
}

int m3probe_write(void* dst, size_t bytes, int blocks, void* stream) {
  hipLaunchKernelGGL(probe_write, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(dst), bytes / 16, 0x3f800000u);
  return (int)hipGetLastError();
}

int m3probe_copy(void* dst, const void* src, size_t bytes, int blocks, void* stream) {
  hipLaunchKernelGGL(probe_copy, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
