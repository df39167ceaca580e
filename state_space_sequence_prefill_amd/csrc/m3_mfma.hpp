// MFMA fragment, conversion and prefetch helpers shared by the prefill kernels.
#pragma once

#include "m3_device.hpp"

namespace m3 {

// ----------------------------------------------------------------------------
// MFMA fragments: 8 K-values per lane for a 16 x 32 (A) or 32 x 16 (B) slab.
// bf16: one v_mfma_f32_16x16x32_bf16.  f32: eight v_mfma_f32_16x16x4_f32, the
// kk-th using element kk of every lane (any K order works as long as the A and
// B fragments agree, which every caller guarantees).
// ----------------------------------------------------------------------------
template <typename IO> struct Frag;
template <> struct Frag<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void set(int k, float f) { v[k] = (bf16)f; }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (bf16)0.0f;
  }
  __device__ __forceinline__ void load8(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ void load44(const bf16* p0, const bf16* p1) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  }
};
template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void set(int k, float f) { v[k] = f; }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.0f;
  }
  __device__ __forceinline__ void load8(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void load44(const float* p0, const float* p1) {
    const float4 a = *reinterpret_cast<const float4*>(p0);
    const float4 b = *reinterpret_cast<const float4*>(p1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int k = 0; k < 8; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[k], b.v[k], acc, 0, 0, 0);
}

// 8 consecutive I/O elements <-> fp32.
__device__ __forceinline__ void load8f(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8f(const bf16* p, float (&o)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(w[k] << 16);
    o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(bf16* p, const float (&v)[8]) {
  bf16x8 o;
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = (bf16)v[k];
  *reinterpret_cast<bf16x8*>(p) = o;
}

// Trig of the chunk-local angles.  bf16 I/O rounds the rotated operands to
// bf16 anyway, so the hardware sin/cos is ample (on angles of any size:
// sincos_hw reduces them first); fp32 I/O uses sincosf.
template <typename IO> __device__ __forceinline__ void trig(float a, float& s, float& c) {
  sincosf(a, &s, &c);
}
template <> __device__ __forceinline__ void trig<bf16>(float a, float& s, float& c) {
  sincos_hw(a, s, c);
}

// 8 consecutive I/O elements as raw 32-bit words (4 for bf16, 8 for fp32).
template <typename IO> struct Raw8 {
  static constexpr int W = 8 * sizeof(IO) / 4;
  uint32_t w[W];
  __device__ __forceinline__ void load(const IO* p) {
#pragma unroll
    for (int k = 0; k < W; k += 4) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[k / 4];
      w[k] = v.x; w[k + 1] = v.y; w[k + 2] = v.z; w[k + 3] = v.w;
    }
  }
  __device__ __forceinline__ void unpack(float (&o)[8]) const {
    if constexpr (sizeof(IO) == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[2 * k] = __uint_as_float(w[k] << 16);
        o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = __uint_as_float(w[k]);
    }
  }
  // Sum of the squares of the 8 elements, straight from the raw words (bf16:
  // v_dot2c_f32_bf16 on each pair, exact products, fp32 sums), so no
  // unpacked copies are formed that the compiler could keep alive for a
  // later unpack of the same registers.
  __device__ __forceinline__ float sumsq() const {
    float s = 0.f;
    if constexpr (sizeof(IO) == 2) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w[k]);
        s = __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) s = fmaf(__uint_as_float(w[k]), __uint_as_float(w[k]), s);
    }
    return s;
  }
};


}  // namespace m3
