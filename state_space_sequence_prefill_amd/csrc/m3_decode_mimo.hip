// Mamba-3 single-token decode step for rank R >= 2 (MIMO) on the matrix cores.
//
// Same update as the VALU kernel in m3_decode.hip (lilting.ch Mamba-3 article,
// "1. 指数台形離散化", "2. 複素数値状態", "3. MIMO SSM"):
//     h <- alpha Rot(theta) h + sum_r x_prev[r] (x) beta Rot(theta) B_prev[r]
//                             + sum_r x[r] (x) gamma B[r]
//     y[r] = h . C[r] + D x[r];   (B_prev, x_prev) <- (B, x)
// The article's MIMO section describes the rank-r coupling as what raises the
// decode step's arithmetic intensity; here both rank contractions run on
// v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate):
//   - the update is a rank-2R product  dh^T = B'^T X'^T  (K = 2R slots: the
//     R pending pairs and the R current ones, in groups of 4);
//   - the readout is  Y^T = C h^T  (K = N, rows r < R of a 16-row tile).
// The state is held as h^T tiles (16 state columns n x 16 rows p) in the MFMA
// accumulator layout: lane (g, c) owns h[p = c][n = 4g .. 4g+3] of its tile,
// which is one 16-byte load and store of the row-major state, and its four
// values are exactly the K operand the readout product needs, so the state
// never moves between lanes.  The rotation acts on column pairs inside a lane.
//
// One workgroup per (b, h); wave w owns state rows p in [16w, 16w + 16) and
// every column tile, so no cross-wave reduction is needed.  The per-head
// operands (pending pair, token, angles) are staged once in LDS, and the
// scaled/rotated rank operands are derived there in fp32 by the workgroup.
#include "m3_device.hpp"
#include "m3_kernels.hpp"

namespace m3 {
namespace {

typedef float f32x4m __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4m __attribute__((ext_vector_type(4)));  // (a vector type, so the staging array stays in registers)

template <typename IO, int N, int R>
struct MimoLds {
  static constexpr int kK = 2 * R;                 // update K slots
  static constexpr int kKG = (kK + 3) / 4;          // MFMA K groups of 4
  // raw staging (I/O dtype): B_prev, B, C (R x N each), x_prev, x (R x P each), theta (N/2 fp32)
  __host__ __device__ static constexpr int granules(int P) {
    return (3 * R * N + 2 * R * P) * (int)sizeof(IO) / 16 + N / 8;
  }
  __host__ __device__ static constexpr size_t raw_bytes(int P) { return (size_t)granules(P) * 16; }
  // derived (fp32): CS[N/2] float2, Bk[4 kKG][N], Xk[4 kKG][P], C[R][N]
  __host__ __device__ static constexpr size_t bytes(int P) {
    return raw_bytes(P) + (size_t)N * 4 + (size_t)4 * kKG * N * 4 + (size_t)4 * kKG * P * 4 + (size_t)R * N * 4;
  }
  // state staging: the P x N fp32 state passes through LDS (rows padded by 4
  // floats) between coalesced HBM runs and the MFMA lane layout
  static constexpr int kLdSt = N + 4;
  __host__ __device__ static constexpr size_t stage_bytes(int P) { return (size_t)P * kLdSt * 4; }
  // BC-norm scales of the 3R rows B_prev, B, C, in whole 64-byte blocks
  static constexpr size_t kSclBytes = ((size_t)3 * R * 4 + 63) / 64 * 64;
  // everything: derived operands, BC-norm scales, staging, gated outputs
  __host__ __device__ static constexpr size_t total_bytes(int P, bool gated) {
    return bytes(P) + kSclBytes + stage_bytes(P) + (gated ? (size_t)R * P * 4 : 0);
  }
};
constexpr int kMimoMaxGranulesPerThread = 3;

template <typename IO, int N, int R, int KG>
__global__ __launch_bounds__(512) void decode_mimo_kernel(DecodeArgs a, int heads, int P) {
  using L = MimoLds<IO, N, R>;
  constexpr int NB = N / 16;        // column tiles per wave
  constexpr int kKG = L::kKG;
  extern __shared__ __align__(16) char dsm[];
  const int head = blockIdx.x;
  const int hh = head % heads;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int pb = wave;              // this wave's 16 state rows

  const IO* x = static_cast<const IO*>(a.x) + (size_t)head * R * P;
  const IO* Bc_ = static_cast<const IO*>(a.B) + (size_t)head * R * N;
  const IO* Cc_ = static_cast<const IO*>(a.C) + (size_t)head * R * N;
  IO* Bp_ = static_cast<IO*>(a.B_prev) + (size_t)head * R * N;
  IO* xp_ = static_cast<IO*>(a.x_prev) + (size_t)head * R * P;
  // this wave's 16 state rows are 16 N contiguous floats: they move between
  // HBM and the LDS staging rows in whole 1 KiB runs (lane l, run j: float4
  // l + 64 j), and between staging and registers in the MFMA layout
  float* const hwave = a.h + (size_t)head * P * N + (size_t)(16 * pb) * N;
  float* const sSt = reinterpret_cast<float*>(dsm + L::bytes(P) + L::kSclBytes) + (size_t)(16 * pb) * L::kLdSt;
  auto stage_off = [&](int j) {  // staging offset of float4 lane + 64 j of the wave's rows
    const int f = lane + 64 * j;
    return (f / (N / 4)) * L::kLdSt + 4 * (f % (N / 4));
  };

  // ---- 1. operand granules, then the state tiles (vmcnt retires in order:
  //         the wait below covers the operands, the state stays in flight)
  const float dt = a.dt[head];
  const float lam = a.lam[head];
  const float Ah = a.A[hh];
  const float Dh = a.D[hh];
  constexpr int gB = R * N * (int)sizeof(IO) / 16;
  const int gX = R * P * (int)sizeof(IO) / 16;
  const int gAll = L::granules(P);
  const u32x4m* const gsrc[6] = {reinterpret_cast<const u32x4m*>(Bp_), reinterpret_cast<const u32x4m*>(Bc_),
                                  reinterpret_cast<const u32x4m*>(Cc_), reinterpret_cast<const u32x4m*>(xp_),
                                  reinterpret_cast<const u32x4m*>(x),
                                  reinterpret_cast<const u32x4m*>(a.theta + (size_t)head * (N / 2))};
  const int gstart[6] = {0, gB, 2 * gB, 3 * gB, 3 * gB + gX, 3 * gB + 2 * gX};
  // output epilogue operands first: the wait below then covers them as well
  const bool gated = a.gz != nullptr;
  DecodeGate<IO, R> gate;
  if (gated)
    gate.prefetch(static_cast<const IO*>(a.gz) + (size_t)head * (a.gdown ? 1 : R) * P, a.gw + (size_t)hh * P,
                  a.gdown ? a.gdown + (size_t)hh * R * P : nullptr, P, wave, nthr / kWave, lane);
  // BC normalisation: when N divides the thread count every element a thread
  // derives in step 2 has column tid % N, so its three weights (the rotation
  // pair of B and the C column) are fetched here, ahead of the barriers
  const bool bcn = a.nbw != nullptr;
  const bool wpre = bcn && nthr % N == 0;
  float wb0, wb1, wc;
  {
    const int n = tid % N;
    const float* nb = wpre ? a.nbw + (size_t)hh * N : a.A;  // (a valid dummy address otherwise)
    const float* nc = wpre ? a.ncw + (size_t)hh * N : a.A;
    wb0 = nb[wpre ? (n & ~1) : 0];
    wb1 = nb[wpre ? (n | 1) : 0];
    wc = nc[wpre ? n : 0];
  }
  // KG granules per thread in registers; KG = 0: more granules than a
  // register array holds, staged by a plain loop first
  auto granule_src = [&](int e) {
    const u32x4m* src = gsrc[0] + e;
#pragma unroll
    for (int q = 1; q < 6; ++q) src = e >= gstart[q] ? gsrc[q] + (e - gstart[q]) : src;
    return src;
  };
  if constexpr (KG == 0) {
    for (int e = tid; e < gAll; e += nthr) reinterpret_cast<u32x4m*>(dsm)[e] = *granule_src(e);
  }
  constexpr int KGR = KG > 0 ? KG : 1;
  u32x4m gv[KGR];
  if constexpr (KG > 0) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      int e = tid + k * nthr;
      e = e < gAll ? e : gAll - 1;  // clamped duplicate, not stored
      gv[k] = *granule_src(e);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float4 hv[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) hv[j] = *reinterpret_cast<const float4*>(hwave + 4 * (lane + 64 * j));
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (KG > 0) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int e = tid + k * nthr;
      if (e < gAll) reinterpret_cast<u32x4m*>(dsm)[e] = gv[k];
    }
  }
  // the old pending pair is read once the operand loads retired (at most NB
  // loads, the state's, outstanding); after the barrier it may be overwritten
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(NB));
  __syncthreads();

  const IO* sBp = reinterpret_cast<const IO*>(dsm);
  const IO* sBc = sBp + R * N;
  const IO* sCc = sBc + R * N;
  const IO* sXp = sCc + R * N;
  const IO* sXc = sXp + R * P;
  const float* sTh = reinterpret_cast<const float*>(sXc + R * P);
  float2* sCS = reinterpret_cast<float2*>(dsm + L::raw_bytes(P));
  float* sBk = reinterpret_cast<float*>(sCS + N / 2);     // [4 kKG][N]
  float* sXk = sBk + 4 * kKG * N;                          // [4 kKG][P]
  float* sCf = sXk + 4 * kKG * P;                          // [R][N]

  // ---- 1b. BC normalisation: RMS scales of the 3R rows B_prev, B, C (wave w
  //          takes rows w, w + waves, ...; lane l columns l and l + 64)
  float* const sScl = reinterpret_cast<float*>(dsm + L::bytes(P));  // [3R], in kSclBytes
  if (bcn) {
    const int nw = nthr / kWave;
    for (int j = wave; j < 3 * R; j += nw) {
      const IO* row = sBp + j * N;  // B_prev, B, C rows are contiguous
      float ss = 0.f;
      for (int n = lane; n < N; n += kWave) {
        const float v = to_f32(row[n]);
        ss += v * v;
      }
      ss = wave_sum(ss);
      if (lane == 0) sScl[j] = rsqrtf(ss * (1.0f / N) + a.neps);
    }
    __syncthreads();
  }
  // the state runs into the staging rows (visible after the next barrier)
#pragma unroll
  for (int j = 0; j < NB; ++j) *reinterpret_cast<float4*>(sSt + stage_off(j)) = hv[j];
  const float* nwB = bcn ? a.nbw + (size_t)hh * N : nullptr;
  const float* nwC = bcn ? a.ncw + (size_t)hh * N : nullptr;

  // ---- 2. derived fp32 operands (whole workgroup)
  {
    const float alpha = expf(dt * Ah);
    const float2 wt = input_weights(dt, lam, alpha, a.disc);
    const float beta = wt.x, gamma = wt.y;
    for (int j = tid; j < N / 2; j += nthr) {
      float s, co;
      sincosf(sTh[j], &s, &co);
      sCS[j] = make_float2(alpha * co, alpha * s);
    }
    // Bk[k][n]: k < R: beta Rot(theta) B_prev[k]; R <= k < 2R: gamma B[k-R]; else 0
    for (int e = tid; e < 4 * kKG * N; e += nthr) {
      const int k = e / N, n = e % N;
      float v = 0.f;
      if (k < R) {
        const int j = n >> 1;
        float s, co;
        sincosf(sTh[j], &s, &co);
        float b0 = to_f32(sBp[k * N + 2 * j]), b1 = to_f32(sBp[k * N + 2 * j + 1]);
        if (bcn) {
          b0 *= (wpre ? wb0 : nwB[2 * j]) * sScl[k];
          b1 *= (wpre ? wb1 : nwB[2 * j + 1]) * sScl[k];
        }
        v = beta * ((n & 1) ? (s * b0 + co * b1) : (co * b0 - s * b1));
      } else if (k < 2 * R) {
        v = gamma * to_f32(sBc[(k - R) * N + n]) * (bcn ? (wpre ? ((n & 1) ? wb1 : wb0) : nwB[n]) * sScl[k] : 1.f);
      }
      sBk[e] = v;
    }
    // Xk[k][p]: k < R: x_prev[k]; R <= k < 2R: x[k-R]; else 0
    for (int e = tid; e < 4 * kKG * P; e += nthr) {
      const int k = e / P, p = e % P;
      sXk[e] = k < R ? to_f32(sXp[k * P + p]) : (k < 2 * R ? to_f32(sXc[(k - R) * P + p]) : 0.f);
    }
    for (int e = tid; e < R * N; e += nthr)
      sCf[e] = to_f32(sCc[e]) * (bcn ? (wpre ? wc : nwC[e % N]) * sScl[2 * R + e / N] : 1.f);
  }
  __syncthreads();

  // ---- 3. per column tile: rotate, rank-2R update on MFMA, store, readout
  float bx[kKG];
#pragma unroll
  for (int q = 0; q < kKG; ++q) bx[q] = sXk[(4 * q + g) * P + 16 * pb + c];
  f32x4m yacc = {0.f, 0.f, 0.f, 0.f};
  // lane (g, c) of tile nb: state row 16 pb + c, columns 16 nb + 4 g .. + 3
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) hv[nb] = *reinterpret_cast<const float4*>(sSt + c * L::kLdSt + 16 * nb + 4 * g);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float4 cs = *reinterpret_cast<const float4*>(sCS + 8 * nb + 2 * g);  // pairs 8nb+2g, +1
    float v[4] = {hv[nb].x, hv[nb].y, hv[nb].z, hv[nb].w};
    rot2(v[0], v[1], cs.x, cs.y);
    rot2(v[2], v[3], cs.z, cs.w);
    f32x4m acc = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int q = 0; q < kKG; ++q)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sBk[(4 * q + g) * N + 16 * nb + c], bx[q], acc, 0, 0, 0);
    *reinterpret_cast<float4*>(sSt + c * L::kLdSt + 16 * nb + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    // readout: K index g <-> n = 16nb + 4g + i for the i-th product
    float4 cr = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < R) cr = *reinterpret_cast<const float4*>(sCf + c * N + 16 * nb + 4 * g);
    yacc = __builtin_amdgcn_mfma_f32_16x16x4f32(cr.x, acc[0], yacc, 0, 0, 0);
    yacc = __builtin_amdgcn_mfma_f32_16x16x4f32(cr.y, acc[1], yacc, 0, 0, 0);
    yacc = __builtin_amdgcn_mfma_f32_16x16x4f32(cr.z, acc[2], yacc, 0, 0, 0);
    yacc = __builtin_amdgcn_mfma_f32_16x16x4f32(cr.w, acc[3], yacc, 0, 0, 0);
  }
  // the new state leaves the staging rows in whole runs
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NB; ++j)
    *reinterpret_cast<float4*>(hwave + 4 * (lane + 64 * j)) = *reinterpret_cast<const float4*>(sSt + stage_off(j));
  // ---- 4. y: lane (g, c) holds Y^T[r = 4g + i][p = 16pb + c], i < 4, for r < R
  //         (gated: the fp32 outputs go to LDS behind the staging rows)
  float* const sYg = reinterpret_cast<float*>(dsm + L::bytes(P) + L::kSclBytes + L::stage_bytes(P));
  if (4 * g < R) {
    IO* y = static_cast<IO*>(a.y) + (size_t)head * R * P + 16 * pb + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      if (r < R) {
        const float xr = sXk[(R + r) * P + 16 * pb + c];
        if (gated)
          sYg[r * P + 16 * pb + c] = yacc[i] + Dh * xr;
        else
          y[r * P] = from_f32<IO>(yacc[i] + Dh * xr);
      }
    }
  }
  // ---- 5. new pending pair from the raw LDS copies, issued last
  for (int e = tid; e < gB + gX; e += nthr) {
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

template <typename IO, int N, int R>
hipError_t launch_mimo_t(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  const int waves = d.P / 16;
  const dim3 grid(d.batch * d.heads), block(waves * kWave);
  const size_t lds = MimoLds<IO, N, R>::total_bytes(d.P, a.gz != nullptr);
  static bool attr_set = false;
  if (!attr_set) {
    for (const void* f : {reinterpret_cast<const void*>(&decode_mimo_kernel<IO, N, R, 1>),
                          reinterpret_cast<const void*>(&decode_mimo_kernel<IO, N, R, kMimoMaxGranulesPerThread>),
                          reinterpret_cast<const void*>(&decode_mimo_kernel<IO, N, R, 0>)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  const int gr = MimoLds<IO, N, R>::granules(d.P);
  if (gr <= waves * kWave)
    hipLaunchKernelGGL((decode_mimo_kernel<IO, N, R, 1>), grid, block, lds, s, a, d.heads, d.P);
  else if (gr <= kMimoMaxGranulesPerThread * waves * kWave)
    hipLaunchKernelGGL((decode_mimo_kernel<IO, N, R, kMimoMaxGranulesPerThread>), grid, block, lds, s, a,
                       d.heads, d.P);
  else
    hipLaunchKernelGGL((decode_mimo_kernel<IO, N, R, 0>), grid, block, lds, s, a, d.heads, d.P);
  return hipGetLastError();
}

template <typename IO, int N>
hipError_t launch_mimo_r(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  switch (d.R) {
    case 2: return launch_mimo_t<IO, N, 2>(d, a, s);
    case 3: return launch_mimo_t<IO, N, 3>(d, a, s);
    case 4: return launch_mimo_t<IO, N, 4>(d, a, s);
    case 5: return launch_mimo_t<IO, N, 5>(d, a, s);
    case 6: return launch_mimo_t<IO, N, 6>(d, a, s);
    case 7: return launch_mimo_t<IO, N, 7>(d, a, s);
    default: return launch_mimo_t<IO, N, 8>(d, a, s);
  }
}

template <typename IO>
hipError_t launch_mimo_n(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  switch (d.N) {
    case 16: return launch_mimo_r<IO, 16>(d, a, s);
    case 32: return launch_mimo_r<IO, 32>(d, a, s);
    case 64: return launch_mimo_r<IO, 64>(d, a, s);
    case 128: return launch_mimo_r<IO, 128>(d, a, s);
    default: return launch_mimo_r<IO, 256>(d, a, s);
  }
}

template <typename IO>
size_t mimo_lds_bytes(int P, int N, int R) {
  switch (N * 16 + R) {
#define M3_CASE(NN, RR) \
  case NN * 16 + RR: return MimoLds<IO, NN, RR>::total_bytes(P, true);
#define M3_CASE_N(NN) M3_CASE(NN, 2) M3_CASE(NN, 3) M3_CASE(NN, 4) M3_CASE(NN, 5) M3_CASE(NN, 6) \
  M3_CASE(NN, 7) M3_CASE(NN, 8)
    M3_CASE_N(16) M3_CASE_N(32) M3_CASE_N(64) M3_CASE_N(128) M3_CASE_N(256)
#undef M3_CASE_N
#undef M3_CASE
    default: return (size_t)-1;
  }
}

}  // namespace

bool decode_mimo_supported(const Dims& d) {
  // rank 1 stays on the VALU kernel (measured faster: its readout would use
  // one row of sixteen in the matrix product); ranks 2 to 8 (the update's
  // 2R slots in up to four K groups, the readout's R rows of a 16-row tile)
  if (!(d.R >= 2 && d.R <= 8)) return false;
  if (!(d.N == 16 || d.N == 32 || d.N == 64 || d.N == 128 || d.N == 256)) return false;
  if (!(d.P == 16 || d.P == 32 || d.P == 64 || d.P == 128)) return false;
  // the staging rows, operands and (gated) outputs in 160 KiB of LDS
  return (d.bf16 ? mimo_lds_bytes<bf16>(d.P, d.N, d.R) : mimo_lds_bytes<float>(d.P, d.N, d.R)) <= 160 * 1024;
}

hipError_t launch_decode_mimo(const Dims& d, const DecodeArgs& a, hipStream_t s) {
  return d.bf16 ? launch_mimo_n<bf16>(d, a, s) : launch_mimo_n<float>(d, a, s);
}

}  // namespace m3
