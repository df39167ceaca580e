// Device-side helpers shared by the gfx950 kernels of the Mamba-3 scan library.
//
// Storage types: I/O tensors are either fp32 (float) or bf16 (__bf16, bit
// pattern of the upper half of an fp32).  All arithmetic is fp32; conversions
// to bf16 round to nearest even (gfx950 v_cvt_pk_bf16_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// Load 4 consecutive I/O elements (16 B for fp32, 8 B for bf16) as fp32.
__device__ __forceinline__ void load4(const float* p, float (&o)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load4(const bf16* p, float (&o)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
}

// Store 4 fp32 values as 4 consecutive I/O elements.
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16* p, const float (&v)[4]) {
  bf16x4 o;
  o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = o;
}

// One 16-byte granule of I/O elements (4 fp32 or 8 bf16) as fp32 values.
template <typename IO> struct Gran;
template <> struct Gran<float> {
  static constexpr int kN = 4;
  __device__ static __forceinline__ void unpack(const uint4& g, float (&o)[4]) {
    o[0] = __uint_as_float(g.x); o[1] = __uint_as_float(g.y);
    o[2] = __uint_as_float(g.z); o[3] = __uint_as_float(g.w);
  }
  __device__ static __forceinline__ uint4 pack(const float (&v)[4]) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
  }
};
template <> struct Gran<bf16> {
  static constexpr int kN = 8;
  __device__ static __forceinline__ void unpack(const uint4& g, float (&o)[8]) {
    const uint32_t w[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ uint4 pack(const float (&v)[8]) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
    return __builtin_bit_cast(uint4, o);
  }
};

// Pair rotation by (c, s): (a, b) -> (a c - b s, a s + b c).
__device__ __forceinline__ void rot2(float& a, float& b, float c, float s) {
  const float na = a * c - b * s;
  const float nb = a * s + b * c;
  a = na;
  b = nb;
}

// Previous- and current-input weights (beta, gamma) of one token under the
// discretisation rule `disc` (m3_disc); alpha = exp(dt A) of the same token.
// lilting.ch Mamba-3 article, "1. 指数台形離散化": Mamba-3's rule weights the
// previous input by (1-lam) dt and the current one by lam dt; the textbook
// trapezoid also decays the previous input by alpha; Mamba-2's exponential
// Euler step keeps only the current input, weighted by dt.
__device__ __forceinline__ float2 input_weights(float dt, float lam, float alpha, int disc) {
  if (disc == 2) return make_float2(0.0f, dt);
  const float b = (1.0f - lam) * dt;
  return make_float2(disc == 1 ? alpha * b : b, lam * dt);
}

// Floor on a token's log-decay dt*A inside the chunked kernels: lower values
// are raised to it before the in-chunk prefix sums.  Such a token (a state
// reset) then passes e^-32 ~ 1.3e-14 of what came before it instead of less:
// the change to any result is below 1.3e-14 times the magnitude of the state
// it erases, far under fp32 resolution.  What the floor buys is precision:
// the prefix sums are rounded relative to their size, and a reset with
// dt*A = -1000 would otherwise leave every later difference of two prefix
// sums with an absolute error of ~1e-4 (~4e-6 with the floor).  It also
// keeps every exponent the kernels form finite.
constexpr float kLogDecayFloor = -32.0f;
__device__ __forceinline__ float log_decay(float dt, float A) { return fmaxf(dt * A, kLogDecayFloor); }

// Sine and cosine of an angle of any size on the hardware units: the angle
// is turned into revolutions, reduced to [0, 1) (an exact operation), and
// passed to v_sin_f32 / v_cos_f32, whose own input domain is +-256
// revolutions.  Error ~1e-6 plus the rounding of a / 2pi (2^-24 |a| / 2pi
// revolutions): ample where the rotated operands are rounded to bf16.
__device__ __forceinline__ void sincos_hw(float a, float& s, float& c) {
  const float r = __builtin_amdgcn_fractf(a * 0.15915494309189535f);
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}

// An angle reduced to about [-pi, pi]: the nearest multiple k of 2 pi is
// subtracted in two parts, an 8-bit head (k * head is exact for |k| < 2^16)
// and the tail.  The chunk-local angle sums of the fp32 kernels then stay
// small enough that their rounding does not show.
__device__ __forceinline__ float reduce_angle(float a) {
  const float k = rintf(a * 0.15915494309189535f);
  const float r = fmaf(-k, 6.28125f, a);
  return fmaf(-k, 1.9353071795864769e-3f, r);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// (0 <= n < 64) are outstanding and leaves the other counters alone: vmcnt
// is split over bits 3:0 and 15:14, expcnt (6:4) and lgkmcnt (11:8) at max.
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Lane-crossing helpers (wave64).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}
__device__ __forceinline__ float shfl_up(float v, int d) { return __shfl_up(v, d, kWave); }

// DPP move with zero fill: lanes whose source is outside the row (or in a
// disabled row) read 0.  ctrl: 0x110 | n = row_shr:n, 0x142 = row_bcast:15,
// 0x143 = row_bcast:31.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}

// Inclusive prefix sum within each row of 16 lanes (4 DPP adds, no LDS).
__device__ __forceinline__ float row16_inclusive_scan(float v) {
  v += dpp_zero<0x111, 0xf>(v);
  v += dpp_zero<0x112, 0xf>(v);
  v += dpp_zero<0x114, 0xf>(v);
  v += dpp_zero<0x118, 0xf>(v);
  return v;
}

// Inclusive prefix sum within each half-wave of 32 lanes.
__device__ __forceinline__ float row32_inclusive_scan(float v) {
  v = row16_inclusive_scan(v);
  v += dpp_zero<0x142, 0xa>(v);  // rows 1 and 3 add the last lane of rows 0 and 2
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  v = row32_inclusive_scan(v);
  v += dpp_zero<0x143, 0xc>(v);  // rows 2 and 3 add lane 31
  return v;
}

// Inclusive prefix sum within aligned segments of `width` lanes (power of two
// <= 64): DPP for 16, 32 and 64, shuffles otherwise.
__device__ __forceinline__ float segment_inclusive_scan(float v, int width) {
  if (width == 16) return row16_inclusive_scan(v);
  if (width == 32) return row32_inclusive_scan(v);
  if (width == 64) return wave_inclusive_scan(v);
  const int sub = threadIdx.x & (width - 1);
  for (int d = 1; d < width; d <<= 1) {
    const float u = __shfl_up(v, d, width);
    if (sub >= d) v += u;
  }
  return v;
}

// Sum over aligned groups of `width` consecutive lanes (a power of two <= 64);
// every lane of a group receives the group's sum.  Within a 16-lane row the
// partners come from DPP (quad permutes, half-row and row mirrors: each pairs
// the lower and the upper half of its group, which is all a sum needs).
__device__ __forceinline__ float lane_group_sum(float v, int width) {
  if (width >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, true));
  if (width >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, true));
  if (width >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, true));
  if (width >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, true));
  if (width >= 32) v += __shfl_xor(v, 16, kWave);
  if (width >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Sum over the whole wave, in every lane: the four row sums from DPP, then
// their total from four lane reads (no LDS round trip, unlike the two
// cross-row shuffles).  (r0 + r1) + (r2 + r3) is the value lane_group_sum(v,
// 64) gives every lane (a + b and b + a round alike).  Needs the whole wave
// active.
__device__ __forceinline__ float wave_sum(float v) {
  v = lane_group_sum(v, 16);
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

// The same for a width known only at run time, up to MAXW (<= 16): every
// step is computed and kept or dropped by a select, so the sum compiles
// without branches (a branch per step costs more than the step).
template <int MAXW>
__device__ __forceinline__ float lane_group_sum_upto(float v, int width) {
  static_assert(MAXW <= 16, "DPP steps only");
  if (MAXW >= 2) {
    const float t = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, true));
    v = width >= 2 ? v + t : v;
  }
  if (MAXW >= 4) {
    const float t = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, true));
    v = width >= 4 ? v + t : v;
  }
  if (MAXW >= 8) {
    const float t = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, true));
    v = width >= 8 ? v + t : v;
  }
  if (MAXW >= 16) {
    const float t = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, true));
    v = width >= 16 ? v + t : v;
  }
  return v;
}

// The output epilogue's per-element map: weight * s * inv_rms * silu(z), with
// silu(z) = z / (1 + exp(-z)) from the hardware exp2 and reciprocal (a correctly
// rounded division would cost ten instructions per element).  Both limits are
// exact: exp2 overflows to inf (silu -> 0) or underflows to 0 (silu -> z).
__device__ __forceinline__ float gate_out(float s, float inv_rms, float w, float z) {
  const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
  return w * s * inv_rms * (z * sig);
}

// Output epilogue of a decode step for one head: R rows of P fp32 scan
// outputs sy[r * P + p] (in LDS) -> y, each row normalised by its RMS, scaled
// by the head's weights and gated.  Wave w of nw handles rows w, w + nw, ...;
// lane l channels l and l + 64 (P <= 128).  With the rank down-projection
// (weights dg (R, P) of this head) the R rows are first folded into one row of
// P channels, which wave 0 normalises and gates.  The gate, weight and
// down-projection values are fetched ahead, before the step's own loads
// (every array element is assigned unconditionally, with selects around
// masked loads, so the arrays stay in registers): read at the end, the
// projection weights' load latency was exposed once per head.
template <typename IO, int R>
struct DecodeGate {
  float z[R][2];
  float w[2];
  float dw[R][2];  // down-projection weights of this lane's channels (wave 0)
  __device__ __forceinline__ void prefetch(const IO* zg, const float* wg, const float* dg, int P, int wave, int nw,
                                           int lane) {
    const bool down = dg != nullptr;
#pragma unroll
    for (int k = 0; k < 2; ++k) w[k] = lane + 64 * k < P ? wg[lane + 64 * k] : 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int p = lane + 64 * k;
        const int r = down ? 0 : wave + i * nw;
        const bool ok = p < P && (down ? (i == 0 && wave == 0) : r < R);
        z[i][k] = ok ? to_f32(zg[r * P + p]) : 0.f;
        dw[i][k] = (down && wave == 0 && p < P) ? dg[i * P + p] : 0.f;
      }
    }
  }
  __device__ __forceinline__ void row(float v0, float v1, IO* yr, float eps, int P, int lane, float z0,
                                      float z1) const {
    const float ss = wave_sum(v0 * v0 + v1 * v1);
    const float inv = rsqrtf(ss / (float)P + eps);
    if (lane < P) yr[lane] = from_f32<IO>(gate_out(v0, inv, w[0], z0));
    if (lane + 64 < P) yr[lane + 64] = from_f32<IO>(gate_out(v1, inv, w[1], z1));
  }
  __device__ __forceinline__ void apply(const float* sy, IO* y, bool down, float eps, int P, int wave, int nw,
                                        int lane) const {
    if (down) {
      if (wave == 0) {
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          v0 += lane < P ? dw[r][0] * sy[r * P + lane] : 0.f;
          v1 += lane + 64 < P ? dw[r][1] * sy[r * P + lane + 64] : 0.f;
        }
        row(v0, v1, y, eps, P, lane, z[0][0], z[0][1]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int r = wave + i * nw;
      if (r < R) {  // uniform over the wave
        const float v0 = lane < P ? sy[r * P + lane] : 0.f;
        const float v1 = lane + 64 < P ? sy[r * P + lane + 64] : 0.f;
        row(v0, v1, y + r * P, eps, P, lane, z[i][0], z[i][1]);
      }
    }
  }
};

// Inclusive prefix sums over strided lanes, K independent values at once (so
// each step's K lane reads are in flight together): within each aligned group
// of count*stride lanes (a power of two <= 64), lane base + k*stride adds the
// values of lanes base + k'*stride for k' <= k (stride, count powers of two,
// count <= 32).
template <int K>
__device__ __forceinline__ void strided_inclusive_scan(float (&v)[K], int stride, int count) {
  const int k = ((int)threadIdx.x / stride) & (count - 1);
  const int lane = (int)threadIdx.x & (kWave - 1);
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    const int d = 1 << s;
    if (d < count) {
      const int src = (lane - d * stride) & (kWave - 1);
      float u[K];
#pragma unroll
      for (int q = 0; q < K; ++q)
        u[q] = __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v[q])));
#pragma unroll
      for (int q = 0; q < K; ++q) v[q] += (k >= d) ? u[q] : 0.f;
    }
  }
}

}  // namespace m3
