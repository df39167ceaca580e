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

// Value of the partner lane in the lower/upper half of an aligned group of
// 2m lanes.  Within a 16-lane row the partner comes from a DPP move (no LDS
// round trip): quad permutes for m = 1, 2, the half-row mirror (lane i <-> 7-i)
// for m = 4 and the row mirror (i <-> 15-i) for m = 8; both mirrors pair every
// lane of the lower half with one of the upper half, which is all the
// reduce-scatter below needs.  Larger m use a lane shuffle.
__device__ __forceinline__ float half_partner(float v, int m) {
  const int iv = __float_as_int(v);
  if (m == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xf, 0xf, true));
  if (m == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xf, 0xf, true));
  if (m == 4) return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0x141, 0xf, 0xf, true));
  if (m == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0x140, 0xf, 0xf, true));
  return shfl_xor(v, m);
}

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
          v[i] = keep + half_partner(send, m);
        }
      }
      cnt = half;
      if (up) base += half;
    } else {
      v[0] += half_partner(v[0], m);
      dup |= m;
    }
  }
}

// Four consecutive I/O elements as loaded (raw bits), unpacked to fp32 later.
template <typename IO> struct Raw4;
template <> struct Raw4<bf16> {
  uint2 w;
  __device__ __forceinline__ void load(const bf16* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void store(bf16* p) const { *reinterpret_cast<uint2*>(p) = w; }
  __device__ __forceinline__ void unpack(float (&o)[4]) const {
    o[0] = __uint_as_float(w.x << 16);
    o[1] = __uint_as_float(w.x & 0xffff0000u);
    o[2] = __uint_as_float(w.y << 16);
    o[3] = __uint_as_float(w.y & 0xffff0000u);
  }
};
template <> struct Raw4<float> {
  float4 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void store(float* p) const { *reinterpret_cast<float4*>(p) = w; }
  __device__ __forceinline__ void unpack(float (&o)[4]) const {
    o[0] = w.x; o[1] = w.y; o[2] = w.z; o[3] = w.w;
  }
};

// IT consecutive I/O elements (IT * sizeof(IO) bytes, naturally aligned) as
// loaded, unpacked to fp32 later.
template <typename IO, int IT>
struct RawRun {
  static constexpr int kBytes = IT * (int)sizeof(IO);
  static constexpr int kWords = kBytes < 4 ? 1 : kBytes / 4;
  uint32_t w[kWords];
  __device__ __forceinline__ void load(const IO* p) {
    if constexpr (kBytes == 2) {
      w[0] = *reinterpret_cast<const uint16_t*>(p);
    } else if constexpr (kBytes == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (kBytes == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
      for (int q = 0; q < kWords / 4; ++q) {
        const uint4 v = reinterpret_cast<const uint4*>(p)[q];
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      }
    }
  }
  __device__ __forceinline__ void store(IO* p) const {
    if constexpr (kBytes == 2) {
      *reinterpret_cast<uint16_t*>(p) = (uint16_t)w[0];
    } else if constexpr (kBytes == 4) {
      *reinterpret_cast<uint32_t*>(p) = w[0];
    } else if constexpr (kBytes == 8) {
      *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int q = 0; q < kWords / 4; ++q)
        reinterpret_cast<uint4*>(p)[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
    }
  }
  __device__ __forceinline__ float at(int i) const {
    if constexpr (sizeof(IO) == 2)
      return __uint_as_float((i & 1) ? (w[i / 2] & 0xffff0000u) : (w[i / 2] << 16));
    else
      return __uint_as_float(w[i]);
  }
  __device__ __forceinline__ void unpack(float (&o)[IT]) const {
    if constexpr (sizeof(IO) == 2) {
#pragma unroll
      for (int i = 0; i < IT; ++i)
        o[i] = __uint_as_float((i & 1) ? (w[i / 2] & 0xffff0000u) : (w[i / 2] << 16));
    } else {
#pragma unroll
      for (int i = 0; i < IT; ++i) o[i] = __uint_as_float(w[i]);
    }
  }
};

// Per-head operands staged in LDS: [B_prev | B | C] (R x N each), [x_prev | x]
// (R x P each), theta (N/2 fp32).  The whole block is brought in with one
// 16-byte load per thread instead of every lane fetching its own copies.
template <typename IO, int N, int R>
struct DecOps {
  static constexpr int kBN = R * N;  // elements of one B-like block
  __host__ __device__ static constexpr int granules(int P) {
    return (3 * kBN + 2 * R * P) * (int)sizeof(IO) / 16 + N / 8;
  }
  __host__ __device__ static constexpr size_t bytes(int P) { return (size_t)granules(P) * 16; }
};
constexpr int kDecMaxGranulesPerThread = 3;

template <typename IO, int N, int R, int IT, int KG>
__global__ __launch_bounds__(1024) void decode_kernel(DecodeArgs a, int heads, int P) {
  constexpr int LPR = N / 4;           // lanes per state row, 4 columns (2 pairs) each
  constexpr int RPI = kWave / LPR;     // state rows covered by one wave instruction
  constexpr int RP = R == 3 ? 4 : R;   // ranks padded to a power of two for the readout (rank 3: one zero)
  constexpr int K = IT * RP;           // readout partial sums per lane
  using Ops = DecOps<IO, N, R>;
  extern __shared__ __align__(16) char dsm[];
  const int head = blockIdx.x;         // flattened (b, h)
  const int hh = head % heads;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int n4 = lane % LPR;
  const int rsub = lane / LPR;
  // lane (rsub, n4) of a wave owns rows row0 .. row0+IT-1 (consecutive, so its
  // x values are one short vector read); one wave instruction i covers rows
  // row0 + i of the RPI row slots
  const int row0 = wave * (RPI * IT) + rsub * IT;
  const int nthr = blockDim.x;

  const IO* x = static_cast<const IO*>(a.x) + (size_t)head * R * P;
  const IO* Bc_ = static_cast<const IO*>(a.B) + (size_t)head * R * N;
  const IO* Cc_ = static_cast<const IO*>(a.C) + (size_t)head * R * N;
  IO* Bp_ = static_cast<IO*>(a.B_prev) + (size_t)head * R * N;
  IO* xp_ = static_cast<IO*>(a.x_prev) + (size_t)head * R * P;
  float* hrow = a.h + (size_t)head * P * N + 4 * n4;

  // ---- 1. operand block (one granule per thread), then the state loads.
  //         Issue order matters: the vmcnt counter retires in order, so the
  //         wait before the barrier covers the operands (among them the old
  //         pending pair) and leaves the state stream in flight.
  constexpr int gB = Ops::kBN * (int)sizeof(IO) / 16;
  const int gX = R * P * (int)sizeof(IO) / 16;
  const int gAll = Ops::granules(P);
  const float dt = a.dt[head];
  const float lam = a.lam[head];
  const float Ah = a.A[hh];
  const float Dh = a.D[hh];
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // (a vector type: the staging array stays in registers)
  const u32x4* const gsrc[6] = {reinterpret_cast<const u32x4*>(Bp_), reinterpret_cast<const u32x4*>(Bc_),
                                reinterpret_cast<const u32x4*>(Cc_), reinterpret_cast<const u32x4*>(xp_),
                                reinterpret_cast<const u32x4*>(x),
                                reinterpret_cast<const u32x4*>(a.theta + (size_t)head * (N / 2))};
  const int gstart[6] = {0, gB, 2 * gB, 3 * gB, 3 * gB + gX, 3 * gB + 2 * gX};
  // BC-normalisation weights of this lane's 4 columns, and the output
  // epilogue operands, first: the wait below then covers them as well
  const bool bcn = a.nbw != nullptr;
  float4 gwb = make_float4(1.f, 1.f, 1.f, 1.f), gwc = gwb;
  if (bcn) {
    gwb = *reinterpret_cast<const float4*>(a.nbw + (size_t)hh * N + 4 * n4);
    gwc = *reinterpret_cast<const float4*>(a.ncw + (size_t)hh * N + 4 * n4);
  }
  const bool gated = a.gz != nullptr;
  DecodeGate<IO, R> gate;
  if (gated)
    gate.prefetch(static_cast<const IO*>(a.gz) + (size_t)head * (a.gdown ? 1 : R) * P, a.gw + (size_t)hh * P,
                  a.gdown ? a.gdown + (size_t)hh * R * P : nullptr, P, wave, nthr / kWave, lane);
  // KG granules per thread (the launch picks KG with KG * threads >= total);
  // every load is unconditional (clamped duplicates are not stored).  KG = 0:
  // more granules than a register array holds, staged by a plain loop first.
  auto granule_src = [&](int e) {
    const u32x4* src = gsrc[0] + e;  // segment by selects, no branch around the load
#pragma unroll
    for (int q = 1; q < 6; ++q) src = e >= gstart[q] ? gsrc[q] + (e - gstart[q]) : src;
    return src;
  };
  if constexpr (KG == 0) {
    for (int e = threadIdx.x; e < gAll; e += nthr) reinterpret_cast<u32x4*>(dsm)[e] = *granule_src(e);
  }
  constexpr int KGR = KG > 0 ? KG : 1;
  u32x4 gv[KGR];
  if constexpr (KG > 0) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      int e = threadIdx.x + k * nthr;
      e = e < gAll ? e : gAll - 1;
      gv[k] = *granule_src(e);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the state loads after the operand loads
  float4 hv[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) hv[i] = *reinterpret_cast<const float4*>(hrow + (size_t)(row0 + i) * N);
  __builtin_amdgcn_sched_barrier(0);  // ... and all IT of them issued before the wait
  if constexpr (KG > 0) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int e = threadIdx.x + k * nthr;
      if (e < gAll) reinterpret_cast<u32x4*>(dsm)[e] = gv[k];
    }
  }
  // The old pending pair has been read once the operand loads retired (at
  // most IT loads, the state's, still outstanding); after the barrier every
  // thread may overwrite it, and the LDS operand block is complete.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(IT));
  __syncthreads();

  const IO* sBp = reinterpret_cast<const IO*>(dsm);
  const IO* sBc = sBp + Ops::kBN;
  const IO* sCc = sBc + Ops::kBN;
  const IO* sXp = sCc + Ops::kBN;
  const IO* sXc = sXp + R * P;
  const float* sTh = reinterpret_cast<const float*>(sXc + R * P);

  // ---- 2. per-lane operands at columns 4*n4 .. 4*n4+3 for every rank
  const float alpha = expf(dt * Ah);
  const float2 wt = input_weights(dt, lam, alpha, a.disc);
  const float beta = wt.x, gamma = wt.y;
  const float2 th = *reinterpret_cast<const float2*>(sTh + 2 * n4);
  float s0, c0, s1, c1;
  sincosf(th.x, &s0, &c0);
  sincosf(th.y, &s1, &c1);
  float Bp[R][4], Bn[R][4], Cn[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    load4(sBp + r * N + 4 * n4, Bp[r]);
    load4(sBc + r * N + 4 * n4, Bn[r]);
    load4(sCc + r * N + 4 * n4, Cn[r]);
    if (bcn) {
      // BC normalisation: row sums over the LPR lanes of a state row (each
      // holds 4 of the N columns), then RMS scale and column weights
      auto norm = [&](float (&v)[4], const float4& gw) {
        const float ss = lane_group_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3], LPR);
        const float sc = rsqrtf(ss * (1.0f / N) + a.neps);
        v[0] *= gw.x * sc;
        v[1] *= gw.y * sc;
        v[2] *= gw.z * sc;
        v[3] *= gw.w * sc;
      };
      norm(Bp[r], gwb);
      norm(Bn[r], gwb);
      norm(Cn[r], gwc);
    }
    rot2(Bp[r][0], Bp[r][1], c0, s0);
    rot2(Bp[r][2], Bp[r][3], c1, s1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      Bp[r][k] *= beta;
      Bn[r][k] *= gamma;
    }
  }
  RawRun<IO, IT> xpr[R], xcr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    xpr[r].load(sXp + r * P + row0);
    xcr[r].load(sXc + r * P + row0);
  }

  // ---- 3. state update, store, readout partial sums
  const float ca = alpha * c0, sa = alpha * s0, cb = alpha * c1, sb = alpha * s1;
  float part[K];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i;
    float v[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
    rot2(v[0], v[1], ca, sa);
    rot2(v[2], v[3], cb, sb);
    float xc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float xp = xpr[r].at(i);
      xc[r] = xcr[r].at(i);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] += xp * Bp[r][k] + xc[r] * Bn[r][k];
    }
    *reinterpret_cast<float4*>(hrow + (size_t)row * N) = make_float4(v[0], v[1], v[2], v[3]);
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float acc = 0.0f;
      if (r < R) {
        acc = (n4 == 0) ? Dh * xc[r] : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc += v[k] * Cn[r][k];
      }
      part[i * RP + r] = acc;
    }
  }
  // ---- 4. readout: reduce the partial sums over the lanes of each row
  int base, dup;
  reduce_scatter<K, LPR>(part, n4, base, dup);
  // (gated: the fp32 outputs go to LDS behind the operand block first)
  float* const sYg = reinterpret_cast<float*>(dsm + Ops::bytes(P));
  if ((n4 & dup) == 0) {
    constexpr int kOut = ReduceScatter<K, LPR>::kOut;
    IO* y = static_cast<IO*>(a.y) + (size_t)head * R * P;
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
      const int idx = base + j;
      const int i = idx / RP;
      const int r = idx % RP;
      if (r < R) {
        if (gated)
          sYg[r * P + row0 + i] = part[j];
        else
          y[r * P + row0 + i] = from_f32<IO>(part[j]);
      }
    }
  }
  // ---- 5. new pending pair (B_prev, x_prev) <- (B, x) from the LDS copies,
  //         issued last (a store ahead of the state's use would make that use
  //         wait for the store as well)
  for (int e = threadIdx.x; e < gB + gX; e += nthr) {
    if (e < gB)
      reinterpret_cast<uint4*>(Bp_)[e] = reinterpret_cast<const uint4*>(sBc)[e];
    else
      reinterpret_cast<uint4*>(xp_)[e - gB] = reinterpret_cast<const uint4*>(sXc)[e - gB];
  }
  // ---- 6. output epilogue (pre-gate grouped RMSNorm) over the LDS outputs
  if (gated) {
    __syncthreads();
    gate.apply(sYg, static_cast<IO*>(a.y) + (size_t)head * (a.gdown ? 1 : R) * P,
               a.gdown != nullptr, a.geps, P, wave, nthr / kWave, lane);
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
  const size_t lds = DecOps<IO, N, R>::bytes(d.P) + (a.gz ? (size_t)R * d.P * sizeof(float) : 0);
  const int gr = DecOps<IO, N, R>::granules(d.P);
  if (gr <= waves * kWave)
    hipLaunchKernelGGL((decode_kernel<IO, N, R, IT, 1>), grid, block, lds, s, a, d.heads, d.P);
  else if (gr <= kDecMaxGranulesPerThread * waves * kWave)
    hipLaunchKernelGGL((decode_kernel<IO, N, R, IT, kDecMaxGranulesPerThread>), grid, block, lds, s, a, d.heads,
                       d.P);
  else
    hipLaunchKernelGGL((decode_kernel<IO, N, R, IT, 0>), grid, block, lds, s, a, d.heads, d.P);
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
    case 3: return launch_it<IO, N, 3>(d, a, s);
    default: return launch_it<IO, N, 4>(d, a, s);
  }
}

template <typename IO>
hipError_t launch_n(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  switch (d.N) {
    case 16: return launch_r<IO, 16>(d, a, s);
    case 32: return launch_r<IO, 32>(d, a, s);
    case 64: return launch_r<IO, 64>(d, a, s);
    case 128: return launch_r<IO, 128>(d, a, s);
    default: return launch_r<IO, 256>(d, a, s);
  }
}

// Sizes the VALU kernel serves: ranks 1 to 4 (its per-lane operands and
// partial sums grow with the rank; ranks above 4 run on the matrix cores).
bool decode_valu_supported(const Dims& d) {
  if (!(d.R >= 1 && d.R <= 4)) return false;
  const int it = pick_iters(d.P, d.N);
  const int waves = d.P * d.N / (4 * kWave * it);
  return waves >= 1 && waves <= 16 && waves * 4 * kWave * it == d.P * d.N;
}

}  // namespace

bool decode_supported(const Dims& d) {
  const bool n_ok = d.N == 16 || d.N == 32 || d.N == 64 || d.N == 128 || d.N == 256;
  const bool p_ok = d.P == 16 || d.P == 32 || d.P == 64 || d.P == 128;
  const bool r_ok = d.R >= 1 && d.R <= 8;
  if (!(n_ok && p_ok && r_ok)) return false;
  return decode_mimo_supported(d) || decode_valu_supported(d);
}

hipError_t launch_decode(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  if (decode_mimo_supported(d)) return launch_decode_mimo(d, a, s);
  if (!decode_valu_supported(d)) return hipErrorInvalidValue;  // (the host checks this first)
  return d.bf16 ? launch_n<bf16>(d, a, s) : launch_n<float>(d, a, s);
}

}  // namespace m3
