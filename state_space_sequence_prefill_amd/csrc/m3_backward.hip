// Backward pass of the Mamba-3 scan: support check, workspace layout and the
// launch sequence.  The kernels (and the derivation) are in m3_backward.hpp;
// m3_backward_bf16.hip and m3_backward_f32.hip instantiate them per I/O type.
#include "m3_backward.hpp"

namespace m3 {

hipError_t launch_backward_bf16(const Dims& d, const BackwardArgs& a, const bwd::BwdWs& w, hipStream_t s);
hipError_t launch_backward_f32(const Dims& d, const BackwardArgs& a, const bwd::BwdWs& w, hipStream_t s);

namespace {

// dA, dD per head: the chains' partial sums over the batch, in batch order
__global__ void backward_reduce_kernel(const float* part, float* dA, float* dD, int batch, int H) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float sa = 0.f, sd = 0.f;
  for (int b = 0; b < batch; ++b) {
    sa += part[((size_t)b * H + h) * 2];
    sd += part[((size_t)b * H + h) * 2 + 1];
  }
  dA[h] = sa;
  dD[h] = sd;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

bool pow2_tile(int v) { return v == 16 || v == 32 || v == 64 || v == 128; }

// workspace offsets (bytes), in BwdWs order; the last entry is the total
void ws_offsets(const Dims& d, int seqlen, size_t (&o)[9]) {
  const size_t chains = (size_t)d.batch * d.heads;
  const size_t qu = (size_t)(bwd::kU / d.R);
  const size_t nu = (seqlen + qu - 1) / qu;
  const size_t pn = (size_t)d.P * d.N;
  const size_t sz[8] = {chains * nu * pn * 4, chains * nu * pn * 4, chains * pn * 4, chains * nu * 4,
                        chains * nu * d.N * 4, chains * nu * 8, chains * nu * 8, chains * 8};
  o[0] = 0;
  for (int i = 0; i < 8; ++i) o[i + 1] = o[i] + align256(sz[i]);
}

}  // namespace

bool backward_supported(const Dims& d) {
  if (!(d.R == 1 || d.R == 2 || d.R == 4)) return false;
  if (!pow2_tile(d.P) || !pow2_tile(d.N) || d.P * d.N > 8192) return false;
  const bwd::Lay ly(d.P, d.N, d.R, true);
  // the angle gradients and their quarter sums reuse the space of X, dY, G
  return (size_t)ly.total * 4 <= 160 * 1024 && ly.Qu * ly.LDPH + 256 <= ly.oBt - ly.oX;
}

size_t backward_workspace_bytes(const Dims& d, int seqlen) {
  size_t o[9];
  ws_offsets(d, seqlen, o);
  return o[8];
}

hipError_t launch_backward(const Dims& d, const BackwardArgs& a, hipStream_t s) {
  size_t o[9];
  ws_offsets(d, a.seqlen, o);
  char* base = static_cast<char*>(a.ws);
  bwd::BwdWs w;
  w.ckE = reinterpret_cast<float*>(base + o[0]);
  w.ckG = reinterpret_cast<float*>(base + o[1]);
  w.dE0 = reinterpret_cast<float*>(base + o[2]);
  w.uel = reinterpret_cast<float*>(base + o[3]);
  w.ucs = reinterpret_cast<float*>(base + o[4]);
  w.nxt = reinterpret_cast<float*>(base + o[5]);
  w.upart = reinterpret_cast<float*>(base + o[6]);
  w.part = reinterpret_cast<float*>(base + o[7]);
  hipError_t e = d.bf16 ? launch_backward_bf16(d, a, w, s) : launch_backward_f32(d, a, w, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(backward_reduce_kernel, dim3((d.heads + 63) / 64), dim3(64), 0, s, w.part, a.dA, a.dD, d.batch,
                     d.heads);
  return hipGetLastError();
}

}  // namespace m3
