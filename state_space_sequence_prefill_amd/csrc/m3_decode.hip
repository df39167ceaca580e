// Mamba-3 single-token decode step for gfx950.
//
// What it computes (per batch row b, head h): one token of the exponential-
// trapezoid recurrence with rotating state (lilting.ch Mamba-3 article,
// "1. 指数台形離散化", "2. 複素数値状態", "3. MIMO SSM"):
//     h <- alpha Rot(theta) h + sum_r [ x_prev[r] (x) beta Rot(theta) B_prev[r]
//                                      + x[r] (x) gamma B[r] ]
//     y[r] = h . C[r] + D x[r];   (B_prev, x_prev) <- (B, x)
// The pending term is moved through the rotation (Rot acts on the state
// columns, so Rot(beta x_prev (x) B_prev) = x_prev (x) beta Rot(theta) B_prev);
// alpha is folded into the rotation coefficients.
//
// The same article ("MIMO SSM" and the comparison table's decode latency)
// describes decode as memory-bound: the fixed-size state is read and written
// once per token and the rank-R work raises the arithmetic intensity.  The
// kernel is built for that bound: one workgroup per (b, h) streams the fp32
// state row-major in 16-byte vectors (64 lanes cover 1 KiB contiguous per
// instruction), keeps all per-head operands (rotated/scaled B columns, C
// columns) in registers, and reduces the readout over the lanes of a state row
// with a reduce-scatter butterfly (IT*R partial sums in log2(N/4) steps).
#include "m3_device.hpp"
#include "m3_kernels.hpp"

namespace m3 {
namespace {

// Reduce-scatter over the lanes of one state row.  Each lane starts with K
// partial sums; lanes that differ only in bits below LPR end up holding
// disjoint windows [base, base + cnt) of the fully reduced sums.  Bits whose
// step runs after the window has shrunk to one value are plain butterflies:
// those lanes hold duplicates, and `dup` collects their bits.
template <int K, int LPR>
struct ReduceScatter {
  static constexpr int steps_with_split(int k, int lpr) {
    return (k <= 1 || lpr <= 1) ? 0 : 1 + steps_with_split(k / 2, lpr / 2);
  }
  static constexpr int kOut = (K >> steps_with_split(K, LPR)) > 0 ? (K >> steps_with_split(K, LPR)) : 1;
};

template <int K, int LPR>
__device__ __forceinline__ void reduce_scatter(float (&v)[K], int sublane, int& base, int& dup) {
  base = 0;
  dup = 0;
  int cnt = K;
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) {
    if (cnt > 1) {
      const int half = cnt / 2;
      const bool up = (sublane & m) != 0;
#pragma unroll
      for (int i = 0; i < K / 2; ++i) {
        if (i < half) {
          const float send = up ? v[i] : v[i + half];
          const float keep = up ? v[i + half] : v[i];
          v[i] = keep + shfl_xor(send, m);
        }
      }
      cnt = half;
      if (up) base += half;
    } else {
      v[0] += shfl_xor(v[0], m);
      dup |= m;
    }
  }
}

template <typename IO, int N, int R, int IT>
__global__ __launch_bounds__(1024) void decode_kernel(DecodeArgs a, int heads, int P) {
  constexpr int LPR = N / 4;           // lanes per state row, 4 columns (2 pairs) each
  constexpr int RPI = kWave / LPR;     // state rows covered by one wave instruction
  constexpr int K = IT * R;            // readout partial sums per lane
  const int head = blockIdx.x;         // flattened (b, h)
  const int hh = head % heads;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int n4 = lane % LPR;
  const int rsub = lane / LPR;
  const int row0 = wave * (RPI * IT) + rsub;

  const IO* x = static_cast<const IO*>(a.x) + (size_t)head * R * P;
  const IO* Bc_ = static_cast<const IO*>(a.B) + (size_t)head * R * N;
  const IO* Cc_ = static_cast<const IO*>(a.C) + (size_t)head * R * N;
  IO* Bp_ = static_cast<IO*>(a.B_prev) + (size_t)head * R * N;
  IO* xp_ = static_cast<IO*>(a.x_prev) + (size_t)head * R * P;
  float* hrow = a.h + (size_t)head * P * N + 4 * n4;

  const float dt = a.dt[head];
  const float lam = a.lam[head];
  const float alpha = expf(dt * a.A[hh]);
  const float beta = (1.0f - lam) * dt;
  const float gamma = lam * dt;
  const float Dh = a.D[hh];
  const float2 th = *reinterpret_cast<const float2*>(a.theta + (size_t)head * (N / 2) + 2 * n4);
  float s0, c0, s1, c1;
  sincosf(th.x, &s0, &c0);
  sincosf(th.y, &s1, &c1);

  // Per-lane operands at columns 4*n4 .. 4*n4+3 for every rank.
  float Bp[R][4], Bn[R][4], Cn[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    load4(Bp_ + r * N + 4 * n4, Bp[r]);
    load4(Bc_ + r * N + 4 * n4, Bn[r]);
    load4(Cc_ + r * N + 4 * n4, Cn[r]);
    rot2(Bp[r][0], Bp[r][1], c0, s0);
    rot2(Bp[r][2], Bp[r][3], c1, s1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      Bp[r][k] *= beta;
      Bn[r][k] *= gamma;
    }
  }
  float xpv[IT][R], xcv[IT][R];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i * RPI;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      xpv[i][r] = to_f32(xp_[r * P + row]);
      xcv[i][r] = to_f32(x[r * P + row]);
    }
  }
  // Every load of the old pending pair must have returned before this
  // workgroup overwrites it (s_waitcnt with all counters at zero).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // New pending pair (B_prev, x_prev) <- (B, x).  Raw element copies.
  for (int e = threadIdx.x; e < R * N; e += blockDim.x) Bp_[e] = Bc_[e];
  for (int e = threadIdx.x; e < R * P; e += blockDim.x) xp_[e] = x[e];

  const float ca = alpha * c0, sa = alpha * s0, cb = alpha * c1, sb = alpha * s1;
  float part[K];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i * RPI;
    float4* hp = reinterpret_cast<float4*>(hrow + (size_t)row * N);
    const float4 hv = *hp;
    float v[4] = {hv.x, hv.y, hv.z, hv.w};
    rot2(v[0], v[1], ca, sa);
    rot2(v[2], v[3], cb, sb);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] += xpv[i][r] * Bp[r][k] + xcv[i][r] * Bn[r][k];
    *hp = make_float4(v[0], v[1], v[2], v[3]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float acc = (n4 == 0) ? Dh * xcv[i][r] : 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc += v[k] * Cn[r][k];
      part[i * R + r] = acc;
    }
  }
  int base, dup;
  reduce_scatter<K, LPR>(part, n4, base, dup);
  if ((n4 & dup) == 0) {
    constexpr int kOut = ReduceScatter<K, LPR>::kOut;
    IO* y = static_cast<IO*>(a.y) + (size_t)head * R * P;
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
      const int idx = base + j;
      const int i = idx / R;
      const int r = idx % R;
      y[r * P + row0 + i * RPI] = from_f32<IO>(part[j]);
    }
  }
}

// Iterations per lane so that one workgroup (<= 16 waves) covers a head.
int pick_iters(int P, int N) {
  const int per_head_vec4 = P * N / 4;
  int it = per_head_vec4 / (4 * kWave);  // aim for 4 waves
  if (it < 1) it = 1;
  if (it > 8) it = 8;
  return it;
}

template <typename IO, int N, int R, int IT>
hipError_t launch_t(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  const int waves = d.P * N / (4 * kWave * IT);
  const dim3 grid(d.batch * d.heads), block(waves * kWave);
  hipLaunchKernelGGL((decode_kernel<IO, N, R, IT>), grid, block, 0, s, a, d.heads, d.P);
  return hipGetLastError();
}

template <typename IO, int N, int R>
hipError_t launch_it(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  switch (pick_iters(d.P, N)) {
    case 1: return launch_t<IO, N, R, 1>(d, a, s);
    case 2: return launch_t<IO, N, R, 2>(d, a, s);
    case 4: return launch_t<IO, N, R, 4>(d, a, s);
    default: return launch_t<IO, N, R, 8>(d, a, s);
  }
}

template <typename IO, int N>
hipError_t launch_r(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  switch (d.R) {
    case 1: return launch_it<IO, N, 1>(d, a, s);
    case 2: return launch_it<IO, N, 2>(d, a, s);
    default: return launch_it<IO, N, 4>(d, a, s);
  }
}

template <typename IO>
hipError_t launch_n(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  switch (d.N) {
    case 16: return launch_r<IO, 16>(d, a, s);
    case 32: return launch_r<IO, 32>(d, a, s);
    case 64: return launch_r<IO, 64>(d, a, s);
    default: return launch_r<IO, 128>(d, a, s);
  }
}

}  // namespace

bool decode_supported(const Dims& d) {
  const bool n_ok = d.N == 16 || d.N == 32 || d.N == 64 || d.N == 128;
  const bool p_ok = d.P == 16 || d.P == 32 || d.P == 64 || d.P == 128;
  const bool r_ok = d.R == 1 || d.R == 2 || d.R == 4;
  if (!(n_ok && p_ok && r_ok)) return false;
  const int it = pick_iters(d.P, d.N);
  const int waves = d.P * d.N / (4 * kWave * it);
  return waves >= 1 && waves <= 16 && waves * 4 * kWave * it == d.P * d.N;
}

hipError_t launch_decode(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  return d.bf16 ? launch_n<bf16>(d, a, s) : launch_n<float>(d, a, s);
}

}  // namespace m3
