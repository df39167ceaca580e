// Backward pass of the Mamba-3 scan for gfx950: gradients of
//     L = sum_t <dy_t, y_t> + <dh_final, h_T>
// with respect to every input of a prefill (lilting.ch Mamba-3 article,
// "アーキテクチャ改善" 1-3: exponential-trapezoid update, rotating state,
// rank-R coupling; the pages train these layers end to end but print no
// backward pass, so it is the exact derivative of the forward definition).
//
// Every chain (b, h) is cut into units of 64 (token, rank) rows (64 / R
// tokens).  In a unit's own frame (angles phi_t and log-decays l_t counted
// from its first token, B and C rotated back by phi_t) the forward step is
// the masked dual form
//     Y   = (S . M) X + diag(e^l) Ct E^T + D X,        S = Ct Bt^T
//     E'  = Rot(phi_end) [ e^{lE} E + sum_k w_k X_k (x) Bt_k ]
// with E the unit's entry value (its first token's decay and pending term
// applied), M the trapezoid mask and w the state-update weights (the next
// token's decay and previous-input weight folded in).  Both recurrences that
// cross units are linear and act on each (p, rotation pair) on its own:
//     E_{u+1} = Rot(phi_end_u) e^{lE_u} E_u + U_u,    U_u = Rot(phi_end_u) sum_k w_k X_k (x) Bt_k
//     dE_u    = e^{lE_u} G_u + V_u,                   V_u = sum_q e^{l_q} dY_q (x) Ct_q,
//     G_u     = Rot(-phi_end_u) dE_{u+1}
// so the pass is four launches:
//   local   every unit at once: U_u, V_u, the unit's end decay and angle;
//   scan    per chain and state element: E_u forward, G_u backward, dE_0;
//   grad    every unit at once, from E_u and G_u: dX, dB, dC, dtheta, ddt,
//           dlam and the unit's shares of dA and dD;
//   finish  per chain: the entry value's gradients (h0, the pending pair,
//           the first token's alpha and beta), the first-token terms each
//           unit hands to the next, and the sums over units.
// The contractions run on the matrix cores in fp32 (v_mfma_f32_16x16x4_f32)
// from LDS tiles; everything else is fp32 VALU.  Gradients are fp32.  With
// bf16 inputs, x and dy are exact bf16 numbers, so the products whose other
// operand is exact too (dY X^T, X dY^T) run on v_mfma_f32_16x16x32_bf16, and
// the local summaries take their fp32 factor as three exact bf16 parts
// (local_bf_kernel); the results are those of the fp32 products up to the
// order of the fp32 sums.  The local and grad kernels are instantiated per
// (P / 16, N / 16), so that every tile loop has a fixed trip count.
//
// MFMA fragments (16 x 16 x 4, wave64): lane (g = lane / 16, c = lane % 16)
// gives A[i = c][k = g] and B[k = g][j = c] and holds D[i = 4 g + v][j = c]
// in register v.  Every contraction orders its K values as k = 16 s + 4 g + v
// for step (s, v); an accumulator tile then serves unchanged as the A operand
// of a product over its row index (as A^T) and the B operand of one over its
// row index, which is how the masked score tiles feed dX, dB and dC.
#pragma once

#include "m3_device.hpp"
#include "m3_kernels.hpp"

namespace m3 {
namespace bwd {

constexpr int kU = 64;        // (token, rank) rows per unit
constexpr int kBT = 256;      // threads of the local and grad kernels: one wave per 16-row block
constexpr int kScanT = 256;
constexpr int kSmall = 1408;  // floats of per-token scalars and partial sums

// per-token slots: sTk[slot * 64 + t]
enum { kL = 0, kL2, kBe, kGa, kW, kEl, kDt, kLm, kNumTk };
// small region (float offsets)
enum {
  oTk = 0, oDga = kNumTk * 64, oDbe = oDga + 64, oDlc = oDbe + 72, oDw = oDlc + 64, oDlp = oDw + 64,
  oPhA = oDlp + 256, oPhB = oPhA + 64, oGE = oPhB + 256, oRed = oGE + 4, oMisc = oRed + 4, oEnd = oMisc + 16
};
static_assert(oEnd <= kSmall, "small region");
// sMisc: [0] lE, [1] e^{lE}, [2] beta of the next token, [3] has next, [4] dt next, [5] lam next

// LDS layout of a unit (float offsets).  X, dY and G are contiguous: they die
// together, and the per-(token, pair) angle gradients reuse their space.
struct Lay {
  int Qu, NH, LDX, LDB, LDPH;
  int oX, odY, oG, oBt, oCt, oPhi, oSm, total;
  __host__ __device__ constexpr Lay(int P, int N, int R, bool grad)
      : Qu(kU / R), NH(N / 2), LDX(P + 4), LDB(N + 4), LDPH(N / 2 + 1), oX(0), odY(kU * (P + 4)),
        oG(2 * kU * (P + 4)), oBt(2 * kU * (P + 4) + (grad ? P * (N + 4) : 0)),
        oCt(oBt + kU * (N + 4)), oPhi(oCt + kU * (N + 4)), oSm(oPhi + (kU / R) * (N / 2 + 1)),
        total(oSm + kSmall) {}
  // (+4 on the row strides: 16-byte row reads and column reads both spread
  // over the banks)
};

// The unit slots (U/E, V/G) hold a P x N matrix in MFMA fragment order: the
// 16 x 16 tile (s, nb) (rows p = 16 s + 4 g + v, columns n = 16 nb + c) is 64
// lanes (g, c) of 4 consecutive floats (v), tiles in (s, nb) order.  A lane
// of a C-layout accumulator stores or loads its 4 values as one 16-byte run,
// and the scan's (p, pair) updates read and write 32-byte runs.

// Workspace carved by launch_backward.
struct BwdWs {
  float* ckE;    // (chains, units, P x N in fragment order): U_u, then E_u
  float* ckG;    // (chains, units, P x N in fragment order): V_u, then G_u
  float* dE0;    // (chains, P, N): adjoint of the entry value
  float* uel;    // (chains, units): e^{lE_u}
  float* ucs;    // (chains, units, N/2, 2): cos, sin of phi_end_u
  float* nxt;    // (chains, units, 2): ddt, dlam of the next unit's first token
  float* upart;  // (chains, units, 2): the unit's dA, dD
  float* part;   // (chains, 2): the chain's dA, dD
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// K slots of a bf16 16x16x32 product over two p slabs: p = 16 s + 4 g + v and
// 16 (s + 1) + 4 g + v (v = 0..3) of an LDS row of exact bf16 values held as
// fp32 (the conversion is exact); the second run is zero when there is no
// slab s + 1.  Both operands of a product take the same slots.
template <bool kTwo>
__device__ __forceinline__ bf16x8 slab_pair(const float* p) {
  const f32x4 a = ld4(p), b = kTwo ? ld4(p + 16) : zero4();
  bf16x8 o;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    o[v] = (bf16)a[v];
    o[4 + v] = (bf16)b[v];
  }
  return o;
}
__device__ __forceinline__ f32x4 mfma_bf(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = lane_group_sum(v, kWave);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < (int)blockDim.x / kWave; ++w) s += red[w];
  return s;
}

// partial derivatives of (beta, gamma) with respect to dt, lam and A
struct DCoef {
  float bdt, blam, bA, gdt, glam;
};
__device__ __forceinline__ DCoef dcoef(float dt, float lam, float A, int disc) {
  const float al = expf(dt * A);
  if (disc == 2) return {0.f, 0.f, 0.f, 1.f, 0.f};
  if (disc == 1) return {(1.f - lam) * al * (1.f + A * dt), -al * dt, (1.f - lam) * dt * dt * al, lam, dt};
  return {1.f - lam, -dt, 0.f, lam, dt};
}

// Trig of the unit-local angles: the hardware sin/cos for bf16 I/O (as in the
// forward kernels, reduced first so any angle is in its domain), sincosf for
// fp32 I/O.
template <typename IO> __device__ __forceinline__ void trig(float a, float& s, float& c) { sincosf(a, &s, &c); }
template <> __device__ __forceinline__ void trig<bf16>(float a, float& s, float& c) { sincos_hw(a, s, c); }

constexpr float kLog2e = 1.4426950408889634f;
// Log-decay below which a token's own decay gradient is taken as zero:
// e^-24 ~ 3.8e-11 is far under the fp32 rounding of the sums it would be
// computed from (see the token scalars of the grad kernel).
constexpr float kDeadLogDecay = -24.0f;

// The value of the neighbouring lane (lane ^ 1), by DPP.
__device__ __forceinline__ float xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
}

// A unit's per-token inputs (pointers at its first token), loaded into
// registers so that they are in flight with the unit's other loads.
template <int NH>
struct CoefIn {
  static constexpr int n = 64 * NH, it = (n + kBT - 1) / kBT;
  float th[it];
  float dt, lm, dtn, lmn;
  __device__ __forceinline__ void load(const float* DTg, const float* LMg, const float* THg, int H, size_t tokTh,
                                       int L, bool nxt) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < it; ++i) {
      const int e = tid + i * kBT, t = e / NH, j = e % NH;
      th[i] = (e < n && t < L) ? THg[(size_t)t * tokTh + j] : 0.f;
    }
    dt = lm = dtn = lmn = 0.f;
    if (tid < 64) {
      if (tid < L) {
        dt = DTg[(size_t)tid * H];
        lm = LMg[(size_t)tid * H];
      }
      if (nxt) {
        dtn = DTg[(size_t)L * H];
        lmn = LMg[(size_t)L * H];
      }
    }
  }
};

// Per-unit coefficients: wave 0, lane t = token: l_t (and l_t log2 e), beta,
// gamma, w_t, e^{l_t}; the angles' inclusive prefix per pair (wave-wide scans,
// lanes = tokens).  Ends with a barrier.
template <int NH>
__device__ __forceinline__ void unit_coefs(const CoefIn<NH>& in, float Ah, int disc, int L, bool nxt, int Qu,
                                           float* sTk, float* sMisc, float* sPhi) {
  constexpr int LDPH = NH + 1, NW = (NH + 3) / 4;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int i = 0; i < CoefIn<NH>::it; ++i) {
    const int e = tid + i * kBT;
    if (e < Qu * NH) sPhi[(e / NH) * LDPH + e % NH] = reduce_angle(in.th[i]);  // small unit-local sums
  }
  if (wv == 0) {
    const int t = lane;
    const bool v = t < L;
    const float av = in.dt * Ah;
    const float2 bg = input_weights(in.dt, in.lm, expf(av), disc);
    const float l = wave_inclusive_scan((v && t > 0) ? log_decay(in.dt, Ah) : 0.f);
    // the next token's decay and previous-input weight close this unit
    const float an = in.dtn * Ah;
    const float bn = nxt ? input_weights(in.dtn, in.lmn, expf(an), disc).x : 0.f;
    const float lE = __shfl(l, L - 1, kWave) + log_decay(in.dtn, Ah);
    const float l_up = __shfl_down(l, 1, kWave), be_up = __shfl_down(bg.x, 1, kWave);
    float w = 0.f;
    if (v) w = bg.y * expf(lE - l) + (t + 1 < L ? be_up * expf(lE - l_up) : bn);
    sTk[kL * 64 + t] = v ? l : 0.f;
    sTk[kL2 * 64 + t] = v ? l * kLog2e : 0.f;
    sTk[kBe * 64 + t] = v ? bg.x : 0.f;
    sTk[kGa * 64 + t] = v ? bg.y : 0.f;
    sTk[kW * 64 + t] = w;
    sTk[kEl * 64 + t] = v ? expf(l) : 0.f;
    sTk[kDt * 64 + t] = in.dt;
    sTk[kLm * 64 + t] = in.lm;
    if (t == 0) {
      sMisc[0] = lE;
      sMisc[1] = expf(lE);
      sMisc[2] = bn;
      sMisc[3] = nxt ? 1.f : 0.f;
      sMisc[4] = in.dtn;
      sMisc[5] = in.lmn;
    }
  }
  __syncthreads();
  float a[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int j = wv + 4 * i;
    a[i] = (j < NH && lane < Qu) ? sPhi[lane * LDPH + j] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < NW; ++i) a[i] = wave_inclusive_scan(a[i]);
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int j = wv + 4 * i;
    if (j < NH && lane < Qu) sPhi[lane * LDPH + j] = a[i];
  }
  __syncthreads();
}

// Rows of a (token, rank)-major input (R = 1 << rs rows of W per token) in
// registers as fp32, zero past the unit's end.
template <typename IO, int W>
struct RowsIn {
  static constexpr int q4 = W / 4, n = kU * q4, it = (n + kBT - 1) / kBT, LD = W + 4;
  float v[it][4];
  static_assert(n % kBT == 0, "whole rows per pass");
  // unconditional loads (rows past the end re-read row 0 and are zeroed):
  // a load under a branch makes the compiler wait for it before the branch joins
  __device__ __forceinline__ void load(const IO* g, size_t tok, int rs, int L) {
#pragma unroll
    for (int i = 0; i < it; ++i) {
      const int e = threadIdx.x + i * kBT, rho = e / q4, c4 = e % q4;
      const int rr = rho < (L << rs) ? rho : 0;
      load4(g + (size_t)(rr >> rs) * tok + (rr & ((1 << rs) - 1)) * W + 4 * c4, v[i]);
    }
  }
  __device__ __forceinline__ void mask(int rs, int L) {
#pragma unroll
    for (int i = 0; i < it; ++i) {
      const int rho = (threadIdx.x + i * kBT) / q4;
      if (rho >= (L << rs)) v[i][0] = v[i][1] = v[i][2] = v[i][3] = 0.f;
    }
  }
  // into LDS (row stride W + 4); rows past the end as zeros
  __device__ __forceinline__ void store(float* dst, int rs, int L) {
    mask(rs, L);
#pragma unroll
    for (int i = 0; i < it; ++i) {
      const int e = threadIdx.x + i * kBT, rho = e / q4, c4 = e % q4;
      *reinterpret_cast<float4*>(dst + rho * LD + 4 * c4) = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
    }
  }
  // rotated back by the token's angle (Rot(-phi_t)) into LDS; W = N
  template <typename IOT>
  __device__ __forceinline__ void store_rot(float* dst, const float* sPhi, int rs, int L) {
    mask(rs, L);
#pragma unroll
    for (int i = 0; i < it; ++i) {
      const int e = threadIdx.x + i * kBT, rho = e / q4, c4 = e % q4;
      const int t = rho >> rs;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float sn, cs;
        trig<IOT>(sPhi[t * (W / 2 + 1) + 2 * c4 + h], sn, cs);
        const float b0 = v[i][2 * h], b1 = v[i][2 * h + 1];
        v[i][2 * h] = b0 * cs + b1 * sn;
        v[i][2 * h + 1] = -b0 * sn + b1 * cs;
      }
      *reinterpret_cast<float4*>(dst + rho * LD + 4 * c4) = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
    }
  }
};

// B and C rows rotated back with one trig per pair.
template <typename IO, int N>
__device__ __forceinline__ void store_rot2(RowsIn<IO, N>& b, RowsIn<IO, N>& c, const float* sPhi, int rs, int L,
                                           float* db, float* dc) {
  using RI = RowsIn<IO, N>;
  b.mask(rs, L);
  c.mask(rs, L);
#pragma unroll
  for (int i = 0; i < RI::it; ++i) {
    const int e = threadIdx.x + i * kBT, rho = e / RI::q4, c4 = e % RI::q4;
    const int t = rho >> rs;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float sn, cs;
      trig<IO>(sPhi[t * (N / 2 + 1) + 2 * c4 + h], sn, cs);
      const float b0 = b.v[i][2 * h], b1 = b.v[i][2 * h + 1], c0 = c.v[i][2 * h], c1 = c.v[i][2 * h + 1];
      b.v[i][2 * h] = b0 * cs + b1 * sn;
      b.v[i][2 * h + 1] = -b0 * sn + b1 * cs;
      c.v[i][2 * h] = c0 * cs + c1 * sn;
      c.v[i][2 * h + 1] = -c0 * sn + c1 * cs;
    }
    *reinterpret_cast<float4*>(db + rho * RI::LD + 4 * c4) = make_float4(b.v[i][0], b.v[i][1], b.v[i][2], b.v[i][3]);
    *reinterpret_cast<float4*>(dc + rho * RI::LD + 4 * c4) = make_float4(c.v[i][0], c.v[i][1], c.v[i][2], c.v[i][3]);
  }
}

// Sum of 4 in-lane row values over the R = 1 << rs rows of each token; the
// group's sum lands in its first register.
__device__ __forceinline__ void rank_sum4(float (&v)[4], int rs) {
  if (rs >= 1) {
    v[0] += v[1];
    v[2] += v[3];
  }
  if (rs >= 2) v[0] += v[2];
}

// ============================ local ============================
// Two workgroups per unit: which = 0 forms U_u from x and B (and stores the
// unit's end decay and angle), which = 1 forms V_u from dy and C.
template <typename IO, int PB, int NB, int RS>
__global__ __launch_bounds__(kBT) void local_kernel(BackwardArgs a, BwdWs ws, int H, int nu) {
  constexpr int rs = RS;  // log2 of the rank (1, 2, 4 -> 0, 1, 2)
  constexpr int P = 16 * PB, N = 16 * NB, NH = N / 2, LDX = P + 4, LDB = N + 4, LDPH = NH + 1;
  extern __shared__ __align__(16) float sm[];
  const int R = 1 << rs, Qu = kU >> rs;
  const int which = blockIdx.x & 1, unit = blockIdx.x >> 1;
  const int chain = unit / nu, u = unit - chain * nu;
  const int hh = chain % H, b = chain / H;
  const int T = a.seqlen, t0 = u * Qu, L = min(Qu, T - t0);
  const bool nxt = t0 + L < T;
  float* sR = sm;             // rows of x (or dy)
  float* sC = sR + kU * LDX;  // rows of Bt (or Ct)
  float* sPhi = sC + kU * LDB;
  float* sTk = sPhi + Qu * LDPH + oTk;
  float* sMisc = sPhi + Qu * LDPH + oMisc;
  const size_t tokBC = (size_t)H * R * N, tokX = (size_t)H * R * P, tokTh = (size_t)H * NH;
  const size_t tb = ((size_t)b * T + t0) * H + hh;  // (b, t0, h)
  CoefIn<NH> ci;
  ci.load(a.dt + tb, a.lam + tb, a.theta + tb * NH, H, tokTh, L, nxt);
  RowsIn<IO, P> rin;
  rin.load(static_cast<const IO*>(which ? a.dy : a.x) + tb * R * P, tokX, rs, L);
  RowsIn<IO, N> cin;
  cin.load(static_cast<const IO*>(which ? a.C : a.B) + tb * R * N, tokBC, rs, L);
  unit_coefs<NH>(ci, a.A[hh], a.disc, L, nxt, Qu, sTk, sMisc, sPhi);
  rin.store(sR, rs, L);
  cin.template store_rot<IO>(sC, sPhi, rs, L);
  __syncthreads();

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  float wk[16];  // row weights (w, or e^l) of this lane's K values k = 16 s + 4 g + v
  const float* tw = sTk + (which ? kEl : kW) * 64;
#pragma unroll
  for (int i = 0; i < 16; ++i) wk[i] = tw[(16 * (i >> 2) + 4 * g + (i & 3)) >> rs];
  const size_t slot = ((size_t)chain * nu + u) * P * N;
  float* Og = (which ? ws.ckG : ws.ckE) + slot;
  const float* phE = sPhi + (L - 1) * LDPH;
  constexpr int kTiles = PB * NB, kPer = (kTiles + 3) / 4;
#pragma unroll
  for (int ti = 0; ti < kPer; ++ti) {
    const int tile = wv + 4 * ti;
    if (tile >= kTiles) break;
    const int pb = tile / NB, nb = tile % NB;
    f32x4 acc = zero4();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = 16 * (i >> 2) + 4 * g + (i & 3);
      acc = mfma4(wk[i] * sR[k * LDX + 16 * pb + c], sC[k * LDB + 16 * nb + c], acc);
    }
    const int n = 16 * nb + c;
    f32x4 o = acc;
    if (!which) {  // U: each (p, pair) turned by the unit's end angle
      const bool odd = c & 1;
      float sn, cs;
      trig<IO>(phE[n >> 1], sn, cs);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float mine = acc[v], other = xor1(mine);
        const float u0 = odd ? other : mine, u1 = odd ? mine : other;
        o[v] = odd ? u0 * sn + u1 * cs : u0 * cs - u1 * sn;
      }
    }
    reinterpret_cast<f32x4*>(Og)[(size_t)(pb * NB + nb) * 64 + lane] = o;
  }
  if (!which) {
    const size_t us = (size_t)chain * nu + u;
    for (int j = threadIdx.x; j < NH; j += kBT) {
      float sn, cs;
      trig<IO>(phE[j], sn, cs);
      reinterpret_cast<float2*>(ws.ucs)[us * NH + j] = make_float2(cs, sn);
    }
    if (threadIdx.x == 0) ws.uel[us] = sMisc[1];
  }
}

// ======================== local, bf16 inputs ========================
// The same U_u and V_u on the bf16 matrix cores.  bf16 inputs are exact bf16
// numbers, so x (or dy) enters v_mfma_f32_16x16x32_bf16 as it is, and the fp32
// factor w B~ (or e^l C~) as three bf16 parts hi + mid + lo whose sum is that
// fp32 value exactly (each part takes the next 8 bits of the 24-bit
// significand); products of bf16 numbers are exact in fp32 and the sums run
// in fp32, so the three products give the fp32 result at a sixth of the
// matrix-core time of v_mfma_f32_16x16x4_f32.  Both operands sit in LDS
// transposed (K = the unit's 64 rows contiguous): rows of 64 bf16 (128 B)
// whose 16-byte chunks are XOR-swizzled by the row index, so the fragment
// reads (16 rows, one chunk each) spread over the banks.
typedef __bf16 bf16x2l __attribute__((ext_vector_type(2)));

// byte offset of element k of row r in a transposed tile
__device__ __forceinline__ int tt_off(int r, int k) { return r * 128 + ((((k >> 3) ^ r) & 7) << 4) + ((k & 7) << 1); }

// RPT consecutive K values of one row (all in one 16-byte chunk)
template <int RPT>
__device__ __forceinline__ void tt_store(char* base, int r, int k0, const float (&v)[RPT]) {
  char* p = base + tt_off(r, k0);
  if constexpr (RPT == 8) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = o;
  } else if constexpr (RPT == 4) {
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (bf16)v[i];
    *reinterpret_cast<bf16x4*>(p) = o;
  } else if constexpr (RPT == 2) {
    bf16x2l o;
    o[0] = (bf16)v[0];
    o[1] = (bf16)v[1];
    *reinterpret_cast<bf16x2l*>(p) = o;
  } else {
    *reinterpret_cast<bf16*>(p) = (bf16)v[0];
  }
}

// Columns of a (token, rank)-major bf16 input: thread t holds columns
// 4 (t % (W/4)) .. + 3 of the W/16 consecutive rows starting at
// (t / (W/4)) W/16, as raw bf16 pairs (rows past the end re-read row 0).
template <int W>
struct ColsIn {
  static constexpr int CG = W / 4, RPT = kU * CG / kBT;
  static_assert(RPT >= 1 && RPT <= 8 && (kU * CG) % kBT == 0, "rows per thread");
  uint32_t lo[RPT], hi[RPT];
  __device__ __forceinline__ void load(const bf16* g, size_t tok, int rs, int L) {
    const int cg = threadIdx.x % CG, r0 = (threadIdx.x / CG) * RPT;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int rho = r0 + i, rr = rho < (L << rs) ? rho : 0;
      const uint2 w = *reinterpret_cast<const uint2*>(g + (size_t)(rr >> rs) * tok + (rr & ((1 << rs) - 1)) * W + 4 * cg);
      lo[i] = w.x;
      hi[i] = w.y;
    }
  }
  // element e (0..3) of row i as fp32
  __device__ __forceinline__ float get(int i, int e) const {
    const uint32_t w = e < 2 ? lo[i] : hi[i];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

template <int PB, int NB, int RS>
__global__ __launch_bounds__(kBT) void local_bf_kernel(BackwardArgs a, BwdWs ws, int H, int nu) {
  constexpr int rs = RS;  // log2 of the rank
  constexpr int P = 16 * PB, N = 16 * NB, NH = N / 2, LDPH = NH + 1;
  using XC = ColsIn<P>;
  using BC = ColsIn<N>;
  extern __shared__ __align__(16) float sm[];
  char* const sXT = reinterpret_cast<char*>(sm);  // (P rows, 64 K) bf16
  char* const sPL = sXT + P * 128;                 // 3 planes of (N rows, 64 K) bf16: lo, mid, hi
  float* const sPhi = reinterpret_cast<float*>(sPL + 3 * N * 128);
  const int R = 1 << rs, Qu = kU >> rs;
  const int which = blockIdx.x & 1, unit = blockIdx.x >> 1;
  const int chain = unit / nu, u = unit - chain * nu;
  const int hh = chain % H, b = chain / H;
  const int T = a.seqlen, t0 = u * Qu, L = min(Qu, T - t0);
  const bool nxt = t0 + L < T;
  float* sTk = sPhi + Qu * LDPH + oTk;
  float* sMisc = sPhi + Qu * LDPH + oMisc;
  const size_t tokBC = (size_t)H * R * N, tokX = (size_t)H * R * P, tokTh = (size_t)H * NH;
  const size_t tb = ((size_t)b * T + t0) * H + hh;  // (b, t0, h)
  CoefIn<NH> ci;
  ci.load(a.dt + tb, a.lam + tb, a.theta + tb * NH, H, tokTh, L, nxt);
  XC xin;
  xin.load(static_cast<const bf16*>(which ? a.dy : a.x) + tb * R * P, tokX, rs, L);
  BC bin;
  bin.load(static_cast<const bf16*>(which ? a.C : a.B) + tb * R * N, tokBC, rs, L);
  unit_coefs<NH>(ci, a.A[hh], a.disc, L, nxt, Qu, sTk, sMisc, sPhi);

  const int nrow = L << rs;
  {  // x (or dy) transposed, rows past the end as zeros
    const int cg = threadIdx.x % XC::CG, r0 = (threadIdx.x / XC::CG) * XC::RPT;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v[XC::RPT];
#pragma unroll
      for (int i = 0; i < XC::RPT; ++i) v[i] = r0 + i < nrow ? xin.get(i, e) : 0.f;
      tt_store<XC::RPT>(sXT, 4 * cg + e, r0, v);
    }
  }
  {  // w B~ (or e^l C~) rotated back per token, split into three planes
    const float* tw = sTk + (which ? kEl : kW) * 64;
    const int cg = threadIdx.x % BC::CG, r0 = (threadIdx.x / BC::CG) * BC::RPT;
    float pv[3][4][BC::RPT];  // [plane][column][row]
#pragma unroll
    for (int i = 0; i < BC::RPT; ++i) {
      const int rho = r0 + i, t = rho >> rs;
      const float wt = rho < nrow ? tw[t] : 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float sn, cs;
        trig<bf16>(sPhi[t * LDPH + 2 * cg + h], sn, cs);
        const float b0 = bin.get(i, 2 * h), b1 = bin.get(i, 2 * h + 1);
        const float r2[2] = {wt * (b0 * cs + b1 * sn), wt * (b1 * cs - b0 * sn)};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float vh = (float)(bf16)r2[q];
          const float rem = r2[q] - vh;
          const float vm = (float)(bf16)rem;
          pv[2][2 * h + q][i] = vh;
          pv[1][2 * h + q][i] = vm;
          pv[0][2 * h + q][i] = rem - vm;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) tt_store<BC::RPT>(sPL + q * N * 128, 4 * cg + e, r0, pv[q][e]);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const size_t slot = ((size_t)chain * nu + u) * P * N;
  float* Og = (which ? ws.ckG : ws.ckE) + slot;
  const float* phE = sPhi + (L - 1) * LDPH;
  constexpr int kTiles = PB * NB, kPer = (kTiles + 3) / 4;
#pragma unroll
  for (int ti = 0; ti < kPer; ++ti) {
    const int tile = wv + 4 * ti;
    if (tile >= kTiles) break;
    const int pb = tile / NB, nb = tile % NB;
    const int p = 16 * pb + c, n = 16 * nb + c;
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kc = 4 * ks + g;
      const bf16x8 xa = *reinterpret_cast<const bf16x8*>(sXT + p * 128 + (((kc ^ p) & 7) << 4));
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sPL + (q * N + n) * 128 + (((kc ^ n) & 7) << 4));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bb, acc, 0, 0, 0);
      }
    }
    f32x4 o = acc;
    if (!which) {  // U: each (p, pair) turned by the unit's end angle
      const bool odd = c & 1;
      float sn, cs;
      trig<bf16>(phE[n >> 1], sn, cs);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float mine = acc[v], other = xor1(mine);
        const float u0 = odd ? other : mine, u1 = odd ? mine : other;
        o[v] = odd ? u0 * sn + u1 * cs : u0 * cs - u1 * sn;
      }
    }
    reinterpret_cast<f32x4*>(Og)[(size_t)(pb * NB + nb) * 64 + lane] = o;
  }
  if (!which) {
    const size_t us = (size_t)chain * nu + u;
    for (int j = threadIdx.x; j < NH; j += kBT) {
      float sn, cs;
      trig<bf16>(phE[j], sn, cs);
      reinterpret_cast<float2*>(ws.ucs)[us * NH + j] = make_float2(cs, sn);
    }
    if (threadIdx.x == 0) ws.uel[us] = sMisc[1];
  }
}

// ============================ scan ============================
// One thread per (chain, 4 rows p, rotation pair): E_u forward from the entry
// value, then G_u backward from dh_final; the slots are read (U_u, V_u) and
// overwritten (E_u, G_u) in place, 32 contiguous bytes per thread (fragment
// order).  Loads run kAhead units ahead of the dependent updates.
template <typename IO>
__global__ __launch_bounds__(kScanT) void scan_kernel(BackwardArgs a, BwdWs ws, int H, int P, int N, int R, int nu,
                                                      int bpc) {
  constexpr int kAhead = 4;
  const int chain = blockIdx.x / bpc;
  const int e = (blockIdx.x - chain * bpc) * kScanT + threadIdx.x;
  const int NH = N / 2, PN = P * N, NB = N / 16;
  if (e >= PN / 8) return;
  const int tile = e >> 5, g = (e >> 3) & 3, c = 2 * (e & 7);
  const int p0 = 16 * (tile / NB) + 4 * g, n = 16 * (tile % NB) + c, j = n >> 1;
  const size_t off = ((size_t)tile * 64 + 16 * g + c) * 4;  // (v, n) then (v, n + 1)
  const int hh = chain % H, b = chain / H;
  const float Ah = a.A[hh];
  const size_t tb0 = (size_t)b * a.seqlen * H + hh;
  const float dt0 = a.dt[tb0], lm0 = a.lam[tb0];
  const float al0 = expf(dt0 * Ah), be0 = input_weights(dt0, lm0, al0, a.disc).x;
  const float* h0 = a.h + (size_t)chain * PN;
  const IO* Bp = static_cast<const IO*>(a.B_prev) + (size_t)chain * R * N;
  const IO* Xp = static_cast<const IO*>(a.x_prev) + (size_t)chain * R * P;
  float E0[4], E1[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float u0 = 0.f, u1 = 0.f;
    for (int r = 0; r < R; ++r) {
      const float xv = to_f32(Xp[r * P + p0 + v]);
      u0 += xv * to_f32(Bp[r * N + n]);
      u1 += xv * to_f32(Bp[r * N + n + 1]);
    }
    const float2 hv = *reinterpret_cast<const float2*>(h0 + (size_t)(p0 + v) * N + n);
    E0[v] = al0 * hv.x + be0 * u0;
    E1[v] = al0 * hv.y + be0 * u1;
  }
  float* cE = ws.ckE + (size_t)chain * nu * PN + off;
  float* cG = ws.ckG + (size_t)chain * nu * PN + off;
  const float* uel = ws.uel + (size_t)chain * nu;
  const float2* ucs = reinterpret_cast<const float2*>(ws.ucs) + (size_t)chain * nu * NH + j;
  for (int ub = 0; ub < nu; ub += kAhead) {
    f32x4 U0[kAhead], U1[kAhead];
    float2 cs[kAhead];
    float el[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int uu = min(ub + i, nu - 1);
      U0[i] = *reinterpret_cast<const f32x4*>(cE + (size_t)uu * PN);
      U1[i] = *reinterpret_cast<const f32x4*>(cE + (size_t)uu * PN + 4);
      cs[i] = ucs[(size_t)uu * NH];
      el[i] = uel[uu];
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      if (ub + i < nu) {
        float* o = cE + (size_t)(ub + i) * PN;
        *reinterpret_cast<f32x4*>(o) = f32x4{E0[0], E0[1], E0[2], E0[3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{E1[0], E1[1], E1[2], E1[3]};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float z0 = el[i] * E0[v], z1 = el[i] * E1[v];
          E0[v] = z0 * cs[i].x - z1 * cs[i].y + U0[i][v];
          E1[v] = z0 * cs[i].y + z1 * cs[i].x + U1[i][v];
        }
      }
    }
  }
  float d0[4] = {0.f, 0.f, 0.f, 0.f}, d1[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.dh_final) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float2 hv = *reinterpret_cast<const float2*>(a.dh_final + (size_t)chain * PN + (size_t)(p0 + v) * N + n);
      d0[v] = hv.x;
      d1[v] = hv.y;
    }
  }
  for (int ub = nu - 1; ub >= 0; ub -= kAhead) {
    f32x4 V0[kAhead], V1[kAhead];
    float2 cs[kAhead];
    float el[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int uu = max(ub - i, 0);
      V0[i] = *reinterpret_cast<const f32x4*>(cG + (size_t)uu * PN);
      V1[i] = *reinterpret_cast<const f32x4*>(cG + (size_t)uu * PN + 4);
      cs[i] = ucs[(size_t)uu * NH];
      el[i] = uel[uu];
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      if (ub - i >= 0) {
        f32x4 g0, g1;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          g0[v] = d0[v] * cs[i].x + d1[v] * cs[i].y;  // Rot(-phi_end) dE_{u+1}
          g1[v] = -d0[v] * cs[i].y + d1[v] * cs[i].x;
          d0[v] = el[i] * g0[v] + V0[i][v];
          d1[v] = el[i] * g1[v] + V1[i][v];
        }
        float* o = cG + (size_t)(ub - i) * PN;
        *reinterpret_cast<f32x4*>(o) = g0;
        *reinterpret_cast<f32x4*>(o + 4) = g1;
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v)
    *reinterpret_cast<float2*>(ws.dE0 + (size_t)chain * PN + (size_t)(p0 + v) * N + n) = make_float2(d0[v], d1[v]);
}

// ============================ grad ============================
// The compute of one unit for the wave that owns row block KB (steps 1-6 of
// grad_kernel).  Instantiated per block so that the masked tiles (queries
// before keys) drop out at compile time.
template <typename IO, int PB, int NB, int KB>
__device__ __forceinline__ void grad_body(const BackwardArgs& a, const float* Eg, float* sm, const Lay& ly, int H,
                                          int L, int rs, float Dh, size_t tb) {
  constexpr int P = 16 * PB, N = 16 * NB, NH = N / 2, LDX = P + 4, LDB = N + 4, LDPH = NH + 1;
  const int R = 1 << rs;
  float* sX = sm + ly.oX;
  float* sdY = sm + ly.odY;
  float* sG = sm + ly.oG;
  float* sBt = sm + ly.oBt;
  float* sCt = sm + ly.oCt;
  float* sPhi = sm + ly.oPhi;
  float* ss = sm + ly.oSm;
  float* sTk = ss + oTk;
  const float* tL2 = sTk + kL2 * 64;
  const float* tBe = sTk + kBe * 64;
  const float* tGa = sTk + kGa * 64;
  const float* tW = sTk + kW * 64;
  const float* tEl = sTk + kEl * 64;
  const size_t tokBC = (size_t)H * R * N, tokX = (size_t)H * R * P;
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int nrow = L << rs;

  // ---- 1. scores: S[q][k] = Ct_q . Bt_k, Pm[q][k] = dY_q . X_k for the
  //         16 columns k of this wave's block and every row q ----
  f32x4 S[4], Pm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) S[i] = Pm[i] = zero4();
  // (row blocks qb < KB hold earlier tokens than every column: masked, skipped)
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    const f32x4 bb = ld4(sBt + (16 * KB + c) * LDB + 16 * s + 4 * g);
    f32x4 aa[4];
#pragma unroll
    for (int qb = KB; qb < 4; ++qb) aa[qb] = ld4(sCt + (16 * qb + c) * LDB + 16 * s + 4 * g);
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int qb = KB; qb < 4; ++qb) S[qb] = mfma4(aa[qb][v], bb[v], S[qb]);
  }
  if constexpr (sizeof(IO) == 2) {  // dY and X are exact bf16: one bf16 product per two p slabs
#pragma unroll
    for (int s = 0; s < PB; s += 2) {
      const bf16x8 bb = slab_pair<(PB > 1)>(sX + (16 * KB + c) * LDX + 16 * s + 4 * g);
#pragma unroll
      for (int qb = KB; qb < 4; ++qb)
        Pm[qb] = mfma_bf(slab_pair<(PB > 1)>(sdY + (16 * qb + c) * LDX + 16 * s + 4 * g), bb, Pm[qb]);
    }
  } else {
#pragma unroll
    for (int s = 0; s < PB; ++s) {
      const f32x4 bb = ld4(sX + (16 * KB + c) * LDX + 16 * s + 4 * g);
      f32x4 aa[4];
#pragma unroll
      for (int qb = KB; qb < 4; ++qb) aa[qb] = ld4(sdY + (16 * qb + c) * LDX + 16 * s + 4 * g);
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int qb = KB; qb < 4; ++qb) Pm[qb] = mfma4(aa[qb][v], bb[v], Pm[qb]);
    }
  }

  // ---- 2. mask: M(q, k) = gamma_k e^{l_q - l_k} + beta_{k+1} e^{l_q - l_{k+1}} [k < q]
  //         (token indices); dM = S . Pm gives the pairs' shares of dgamma,
  //         dbeta (column sums) and dl (row sums); S and Pm become M.S, M.Pm ----
  {
    const int tk = (16 * KB + c) >> rs;
    const int tk1 = min(tk + 1, 63);
    const float lk = tL2[tk], lk1 = tL2[tk1], gk = tGa[tk], bk1 = tBe[tk1];
    float cg = 0.f, cb = 0.f;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      if (qb < KB) {  // masked block: no pair terms, zero row sums
#pragma unroll
        for (int v = 0; v < 4; v += R)
          if (c == 0) ss[oDlp + KB * 64 + ((16 * qb + 4 * g + v) >> rs)] = 0.f;
        continue;
      }
      float rl[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tq = (16 * qb + 4 * g + v) >> rs;
        const bool on = tq < L && tk <= tq;
        const float lq = tL2[tq];
        const float e1 = on ? __builtin_amdgcn_exp2f(lq - lk) : 0.f;
        const float e2 = (on && tk < tq) ? __builtin_amdgcn_exp2f(lq - lk1) : 0.f;
        const float m = gk * e1 + bk1 * e2;
        const float sv = S[qb][v], pv = Pm[qb][v], d = sv * pv;
        cg += d * e1;
        cb += d * e2;
        rl[v] = d * m;
        S[qb][v] = m * sv;
        Pm[qb][v] = m * pv;
      }
      rank_sum4(rl, rs);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (v & (R - 1)) continue;
        const float r = lane_group_sum(rl[v], 16);
        if (c == 0) ss[oDlp + KB * 64 + ((16 * qb + 4 * g + v) >> rs)] = r;
      }
    }
    cg += __shfl_xor(cg, 16, kWave);
    cg += __shfl_xor(cg, 32, kWave);
    cb += __shfl_xor(cb, 16, kWave);
    cb += __shfl_xor(cb, 32, kWave);
    cg = lane_group_sum(cg, R);
    cb = lane_group_sum(cb, R);
    if (g == 0 && (c & (R - 1)) == 0) {
      ss[oDga + tk] = cg;
      ss[oDbe + tk + 1] = cb;
    }
  }

  // ---- 3. GB[k][p] = Bt_k . G_p; dw_k = X_k . GB_k;
  //         dX = w GB + D dY + (M.S)^T dY, rows of this wave's block ----
  {
    f32x4 acc[PB];
#pragma unroll
    for (int i = 0; i < PB; ++i) acc[i] = zero4();
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      const f32x4 aa = ld4(sBt + (16 * KB + c) * LDB + 16 * s + 4 * g);
      f32x4 bb[PB];
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) bb[pb] = ld4(sG + (16 * pb + c) * LDB + 16 * s + 4 * g);
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) acc[pb] = mfma4(aa[v], bb[pb][v], acc[pb]);
    }
    float dwv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
      for (int v = 0; v < 4; ++v) dwv[v] += sX[(16 * KB + 4 * g + v) * LDX + 16 * pb + c] * acc[pb][v];
    rank_sum4(dwv, rs);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v & (R - 1)) continue;
      const float r = lane_group_sum(dwv[v], 16);
      if (c == 0) ss[oDw + ((16 * KB + 4 * g + v) >> rs)] = r;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int k = 16 * KB + 4 * g + v;
      const float wr = tW[k >> rs];
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) acc[pb][v] = wr * acc[pb][v] + Dh * sdY[k * LDX + 16 * pb + c];
    }
#pragma unroll
    for (int qb = KB; qb < 4; ++qb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = S[qb][v];
        const float* yr = sdY + (16 * qb + 4 * g + v) * LDX + c;
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) acc[pb] = mfma4(av, yr[16 * pb], acc[pb]);
      }
    float* dXg = a.dx + tb * R * P;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int k = 16 * KB + 4 * g + v;
      if (k < nrow) {
        float* o = dXg + (size_t)(k >> rs) * tokX + (k & (R - 1)) * P + c;
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) o[16 * pb] = acc[pb][v];
      }
    }
  }

  // ---- 4. GX[k][n] = X_k . G[:, n]; dBt = w GX + (M.Pm)^T Ct, rows of this
  //         block; the end angle's share through the update weights ----
  f32x4 db[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) db[i] = zero4();
#pragma unroll
  for (int s = 0; s < PB; ++s) {
    const f32x4 aa = ld4(sX + (16 * KB + c) * LDX + 16 * s + 4 * g);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float* gr = sG + (16 * s + 4 * g + v) * LDB + c;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) db[nb] = mfma4(aa[v], gr[16 * nb], db[nb]);
    }
  }
  {
    float wr[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) wr[v] = tW[(16 * KB + 4 * g + v) >> rs];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = 16 * nb + c;
      float ph = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int k = 16 * KB + 4 * g + v;
        const float gx = db[nb][v], gxo = xor1(gx);
        ph += wr[v] * (sBt[k * LDB + n] * gxo - sBt[k * LDB + (n ^ 1)] * gx);  // even lanes: Bt0 GX1 - Bt1 GX0
      }
      ph += __shfl_xor(ph, 16, kWave);
      ph += __shfl_xor(ph, 32, kWave);
      if (g == 0 && !(c & 1)) ss[oPhB + KB * 64 + (n >> 1)] = ph;
#pragma unroll
      for (int v = 0; v < 4; ++v) db[nb][v] *= wr[v];
    }
  }
#pragma unroll
  for (int qb = KB; qb < 4; ++qb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float av = Pm[qb][v];
      const float* cr = sCt + (16 * qb + 4 * g + v) * LDB + c;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) db[nb] = mfma4(av, cr[16 * nb], db[nb]);
    }

  // E (the unit's entry value) for the carried product of step 5, loaded here
  // (fragment order: lane (g, c) of tile (s, nb) holds E[16 s + 4 g + v][16 nb + c], v = 0..3)
  f32x4 ev[PB][NB];
#pragma unroll
  for (int s = 0; s < PB; ++s)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ev[s][nb] = reinterpret_cast<const f32x4*>(Eg)[(s * NB + nb) * 64 + lane];
  // ---- 5. PmT[k][q] = X_k . dY_q (rows q of this block, every k);
  //         carry[q][n] = dY_q . E[:, n]; dCt = e^l carry + (M.Pm) Bt;
  //         <G, E> and the end angle's share through E ----
  f32x4 dc[NB];
  {
    f32x4 PT[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) PT[i] = zero4();
#pragma unroll
    for (int i = 0; i < NB; ++i) dc[i] = zero4();
    float ge = 0.f, pha[2] = {0.f, 0.f};
    if constexpr (sizeof(IO) == 2) {  // exact bf16 operands, as Pm
#pragma unroll
      for (int s = 0; s < PB; s += 2) {
        const bf16x8 yq = slab_pair<(PB > 1)>(sdY + (16 * KB + c) * LDX + 16 * s + 4 * g);
#pragma unroll
        for (int kb = 0; kb <= KB; ++kb)
          PT[kb] = mfma_bf(slab_pair<(PB > 1)>(sX + (16 * kb + c) * LDX + 16 * s + 4 * g), yq, PT[kb]);
      }
    }
#pragma unroll
    for (int s = 0; s < PB; ++s) {
      const f32x4 yb = ld4(sdY + (16 * KB + c) * LDX + 16 * s + 4 * g);
      if constexpr (sizeof(IO) != 2) {
        f32x4 xa[4];  // (key blocks kb > KB hold later tokens than every query here: masked, skipped)
#pragma unroll
        for (int kb = 0; kb <= KB; ++kb) xa[kb] = ld4(sX + (16 * kb + c) * LDX + 16 * s + 4 * g);
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int kb = 0; kb <= KB; ++kb) PT[kb] = mfma4(xa[kb][v], yb[v], PT[kb]);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) dc[nb] = mfma4(yb[v], ev[s][nb][v], dc[nb]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if ((nb & 3) != KB) continue;  // pair columns nb = KB (mod 4)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int p = 16 * s + 4 * g + v, n = 16 * nb + c;
          const float e = ev[s][nb][v];
          const float eo = xor1(e);
          const float gs = sG[p * LDB + n], go = sG[p * LDB + (n ^ 1)];
          ge += gs * e;
          pha[nb >> 2] += go * e - gs * eo;  // even lanes: G1 E0 - G0 E1
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int nb = KB + 4 * i;
      if (nb >= NB) continue;
      float v = pha[i];
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      if (g == 0 && !(c & 1)) ss[oPhA + ((16 * nb + c) >> 1)] = v;
    }
    ge = lane_group_sum(ge, kWave);
    if (lane == 0) ss[oGE + KB] = ge;
    // carried part of dl: e^{l_q} sum_n carry[q][n] Ct[q][n]
    float dl4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) dl4[v] += dc[nb][v] * sCt[(16 * KB + 4 * g + v) * LDB + 16 * nb + c];
    rank_sum4(dl4, rs);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v & (R - 1)) continue;
      const float r = lane_group_sum(dl4[v], 16);
      const int tq = (16 * KB + 4 * g + v) >> rs;
      if (c == 0) ss[oDlc + tq] = tEl[tq] * r;
    }
    // mask of the transposed tiles: rows k = 16 kb + 4 g + v, column q = 16 KB + c
    {
      const int tq = (16 * KB + c) >> rs;
      const float lq = tL2[tq];
#pragma unroll
      for (int kb = 0; kb <= KB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tk = (16 * kb + 4 * g + v) >> rs, tk1 = min(tk + 1, 63);
          const bool on = tq < L && tk <= tq;
          const float e1 = on ? __builtin_amdgcn_exp2f(lq - tL2[tk]) : 0.f;
          const float e2 = (on && tk < tq) ? __builtin_amdgcn_exp2f(lq - tL2[tk1]) : 0.f;
          PT[kb][v] *= tGa[tk] * e1 + tBe[tk1] * e2;
        }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float el = tEl[(16 * KB + 4 * g + v) >> rs];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) dc[nb][v] *= el;
    }
#pragma unroll
    for (int kb = 0; kb <= KB; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = PT[kb][v];
        const float* br = sBt + (16 * kb + 4 * g + v) * LDB + c;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) dc[nb] = mfma4(av, br[16 * nb], dc[nb]);
      }
  }
  // <dY, X> over the unit (D's gradient)
  {
    float yx = 0.f;
#pragma unroll
    for (int i = 0; i < kU * P / kBT; ++i) {
      const int e = threadIdx.x + i * kBT, rho = e / P, p = e % P;
      yx += sdY[rho * LDX + p] * sX[rho * LDX + p];
    }
    yx = lane_group_sum(yx, kWave);
    if (lane == 0) ss[oRed + KB] = yx;
  }
  __syncthreads();  // X, dY and G are dead: their space takes the angle gradients

  // ---- 6. rows back to the lab frame (dB, dC); angle gradient per (token, pair) ----
  // After the barrier above every wave reads only its own 16 rows of Bt and
  // Ct, so each overwrites them with its dB, dC rows (after reading them for
  // the angle gradient) and writes those rows out as whole 16-byte runs.
  float* sDphi = sm + ly.oX;
  {
    const bool odd = c & 1;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = 16 * nb + c, j = n >> 1;
      float phs[4], ob[4], oc[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * KB + 4 * g + v, t = row >> rs;
        const float bq = db[nb][v], bo = xor1(bq);
        const float cq = dc[nb][v], co = xor1(cq);
        const float d0 = odd ? bo : bq, d1 = odd ? bq : bo;
        const float e0 = odd ? co : cq, e1 = odd ? cq : co;
        float sn, cs;
        trig<IO>(sPhi[t * LDPH + j], sn, cs);
        ob[v] = odd ? d0 * sn + d1 * cs : d0 * cs - d1 * sn;  // Rot(+phi)
        oc[v] = odd ? e0 * sn + e1 * cs : e0 * cs - e1 * sn;
        const float* br = sBt + row * LDB + (n & ~1);
        const float* cr = sCt + row * LDB + (n & ~1);
        phs[v] = d0 * br[1] - d1 * br[0] + e0 * cr[1] - e1 * cr[0];
      }
      // (the wave's reads above precede these writes in its LDS queue)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * KB + 4 * g + v;
        sBt[row * LDB + n] = ob[v];
        sCt[row * LDB + n] = oc[v];
      }
      rank_sum4(phs, rs);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (v & (R - 1)) continue;
        if (!odd) sDphi[((16 * KB + 4 * g + v) >> rs) * LDPH + j] = phs[v];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float* dBg = a.dB + tb * R * N;
    float* dCg = a.dC + tb * R * N;
    constexpr int Q4 = N / 4, kIt = 16 * Q4 / kWave;  // 16-byte runs of the wave's 16 rows, per lane
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int e = lane + kWave * i, row = 16 * KB + e / Q4, q = e % Q4;
      if (row < nrow) {
        const size_t o = (size_t)(row >> rs) * tokBC + (row & (R - 1)) * N + 4 * q;
        *reinterpret_cast<f32x4*>(dBg + o) = ld4(sBt + row * LDB + 4 * q);
        *reinterpret_cast<f32x4*>(dCg + o) = ld4(sCt + row * LDB + 4 * q);
      }
    }
  }
  __syncthreads();

}

// One workgroup per CU (its LDS), one wave per SIMD: the whole register file
// is this wave's.
template <typename IO, int PB, int NB, int RS>
__global__ __launch_bounds__(kBT) __attribute__((amdgpu_waves_per_eu(1, 1))) void grad_kernel(BackwardArgs a, BwdWs ws, int H, int nu) {
  constexpr int rs = RS;  // log2 of the rank
  constexpr int P = 16 * PB, N = 16 * NB, NH = N / 2, LDX = P + 4, LDB = N + 4, LDPH = NH + 1;
  extern __shared__ __align__(16) float sm[];
  const int R = 1 << rs;
  const Lay ly(P, N, R, true);
  const int chain = blockIdx.x / nu, u = blockIdx.x - chain * nu;
  const int hh = chain % H, b = chain / H;
  const int T = a.seqlen, t0 = u * ly.Qu, L = min(ly.Qu, T - t0);
  const bool nxt = t0 + L < T;
  const float Ah = a.A[hh], Dh = a.D[hh];
  float* sX = sm + ly.oX;
  float* sdY = sm + ly.odY;
  float* sG = sm + ly.oG;
  float* sBt = sm + ly.oBt;
  float* sCt = sm + ly.oCt;
  float* sPhi = sm + ly.oPhi;
  float* ss = sm + ly.oSm;
  float* sTk = ss + oTk;
  float* sMisc = ss + oMisc;
  const float* tL = sTk + kL * 64;
  const float* tL2 = sTk + kL2 * 64;
  const float* tBe = sTk + kBe * 64;
  const float* tGa = sTk + kGa * 64;
  const float* tW = sTk + kW * 64;
  const float* tEl = sTk + kEl * 64;
  const size_t tokBC = (size_t)H * R * N, tokX = (size_t)H * R * P, tokTh = (size_t)H * NH;
  const size_t tb = ((size_t)b * T + t0) * H + hh;
  const size_t slot = ((size_t)chain * nu + u) * P * N;
  const float* Eg = ws.ckE + slot;
  const float* Gg = ws.ckG + slot;

  // every global load of the unit in flight together
  CoefIn<NH> ci;
  ci.load(a.dt + tb, a.lam + tb, a.theta + tb * NH, H, tokTh, L, nxt);
  constexpr int n4 = P * N / 4, itG = (n4 + kBT - 1) / kBT;
  f32x4 gv[itG];  // fragment order: float4 e = (tile e / 64, lane e % 64)
#pragma unroll
  for (int i = 0; i < itG; ++i) gv[i] = reinterpret_cast<const f32x4*>(Gg)[min((int)threadIdx.x + i * kBT, n4 - 1)];
  RowsIn<IO, P> xin, yin;
  RowsIn<IO, N> bin, cin;
  xin.load(static_cast<const IO*>(a.x) + tb * R * P, tokX, rs, L);
  yin.load(static_cast<const IO*>(a.dy) + tb * R * P, tokX, rs, L);
  bin.load(static_cast<const IO*>(a.B) + tb * R * N, tokBC, rs, L);
  cin.load(static_cast<const IO*>(a.C) + tb * R * N, tokBC, rs, L);
  unit_coefs<NH>(ci, Ah, a.disc, L, nxt, ly.Qu, sTk, sMisc, sPhi);
#pragma unroll
  for (int i = 0; i < itG; ++i) {
    const int e = threadIdx.x + i * kBT, tile = e >> 6, ln = e & 63;
    float* d = sG + (16 * (tile / NB) + 4 * (ln >> 4)) * LDB + 16 * (tile % NB) + (ln & 15);
    if (e < n4)
#pragma unroll
      for (int v = 0; v < 4; ++v) d[v * LDB] = gv[i][v];
  }
  xin.store(sX, rs, L);
  yin.store(sdY, rs, L);
  store_rot2<IO, N>(bin, cin, sPhi, rs, L, sBt, sCt);
  __syncthreads();

  switch (threadIdx.x >> 6) {
    case 0: grad_body<IO, PB, NB, 0>(a, Eg, sm, ly, H, L, rs, Dh, tb); break;
    case 1: grad_body<IO, PB, NB, 1>(a, Eg, sm, ly, H, L, rs, Dh, tb); break;
    case 2: grad_body<IO, PB, NB, 2>(a, Eg, sm, ly, H, L, rs, Dh, tb); break;
    default: grad_body<IO, PB, NB, 3>(a, Eg, sm, ly, H, L, rs, Dh, tb); break;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float* sDphi = sm + ly.oX;

  // ---- 7. token scalars (wave 0, lane t = token) and angles ----
  const float elE = sMisc[1];
  if (wv == 0) {
    const int t = lane;
    const bool v = t < L;
    const float lE = sMisc[0], bn = sMisc[2];
    float dga = 0.f, dbe = 0.f, dl = 0.f, dwt = 0.f, wpart = 0.f;
    if (v) {
      const float lt = tL[t];
      dwt = ss[oDw + t];
      const float ee = expf(lE - lt);
      dga = ss[oDga + t] + dwt * ee;
      if (t >= 1) dbe = ss[oDbe + t] + ss[oDw + t - 1] * ee;
      const float rsum = ss[oDlp + t] + ss[oDlp + 64 + t] + ss[oDlp + 128 + t] + ss[oDlp + 192 + t];
      dl = ss[oDlc + t] + rsum - tGa[t] * dga - (t >= 1 ? tBe[t] * dbe : 0.f);
      wpart = dwt * (tW[t] - (t == L - 1 ? bn : 0.f));
    }
    const float ge = ss[oGE] + ss[oGE + 1] + ss[oGE + 2] + ss[oGE + 3];
    const float dlE = elE * ge + lane_group_sum(wpart, kWave);
    const float dbn = __shfl(dwt, L - 1, kWave);  // the next token's beta, weight 1
    const float pre = wave_inclusive_scan(dl);
    const float rc = lane_group_sum(dl, kWave) - pre + dl;  // sum_{s >= t} dl_s
    float dAp = 0.f;
    if (v) {
      const float dt = sTk[kDt * 64 + t], lm = sTk[kLm * 64 + t];
      // Every term of the loss that depends on this token's log-decay a_t
      // carries the factor e^{a_t}, so |da_t| <= e^{a_t} times the size of
      // those terms.  Below kDeadLogDecay that is under the rounding noise of
      // the suffix sum (its +M and -M terms of the pairs after the token
      // cancel only to fp32 precision), and the noise times a large dt would
      // swamp dA: such a token's da is zero to fp32 accuracy.
      const float da = (t > 0 && dt * Ah >= kDeadLogDecay) ? rc + dlE : 0.f;
      const DCoef dcf = dcoef(dt, lm, Ah, a.disc);
      a.ddt[tb + (size_t)t * H] = Ah * da + dcf.bdt * dbe + dcf.gdt * dga;
      a.dlam[tb + (size_t)t * H] = dcf.blam * dbe + dcf.glam * dga;
      dAp = dt * da + dcf.bA * dbe;
    }
    dAp = lane_group_sum(dAp, kWave);
    if (t == 0) {
      float nd = 0.f, nl = 0.f;
      if (sMisc[3] != 0.f) {  // the next token's decay and previous-input weight
        const float dtn = sMisc[4], lmn = sMisc[5];
        const DCoef dcn = dcoef(dtn, lmn, Ah, a.disc);
        const float dan = dtn * Ah >= kDeadLogDecay ? dlE : 0.f;  // as da above
        nd = Ah * dan + dcn.bdt * dbn;
        nl = dcn.blam * dbn;
        dAp += dtn * dan + dcn.bA * dbn;
      }
      const size_t us = (size_t)chain * nu + u;
      ws.nxt[us * 2] = nd;
      ws.nxt[us * 2 + 1] = nl;
      ws.upart[us * 2] = dAp;
      ws.upart[us * 2 + 1] = ss[oRed] + ss[oRed + 1] + ss[oRed + 2] + ss[oRed + 3];
    }
  }
  // dtheta_s = sum_{t >= s} dphi_t + dphi_end,
  // dphi_end = e^{lE} sum_p (G1 E0 - G0 E1) + sum_k w_k (Bt0 GX1 - Bt1 GX0);
  // the four waves take a quarter of the tokens each
  {
    float* sDq = sDphi + ly.Qu * LDPH;  // (4, 64) quarter sums
    const int qt = wv, j = lane, Qq = ly.Qu / 4;
    const int ta = qt * Qq, te = min(ta + Qq, L);
    float part = 0.f;
    if (j < NH)
      for (int t = ta; t < te; ++t) part += sDphi[t * LDPH + j];
    sDq[qt * 64 + j] = part;
    __syncthreads();
    if (j < NH) {
      float acc = elE * ss[oPhA + j] + ss[oPhB + j] + ss[oPhB + 64 + j] + ss[oPhB + 128 + j] + ss[oPhB + 192 + j];
      for (int q2 = 3; q2 > qt; --q2) acc += sDq[q2 * 64 + j];
      float* dTHg = a.dtheta + tb * NH + j;
      for (int t = te - 1; t >= ta; --t) {
        acc += sDphi[t * LDPH + j];
        dTHg[(size_t)t * tokTh] = acc;
      }
    }
  }
}

// ============================ finish ============================
template <typename IO>
__global__ __launch_bounds__(256) void finish_kernel(BackwardArgs a, BwdWs ws, int H, int P, int N, int R, int nu) {
  __shared__ float red[8];
  const int chain = blockIdx.x, tid = threadIdx.x;
  const int hh = chain % H, b = chain / H;
  const int T = a.seqlen, Qu = kU / R, PN = P * N;
  const float Ah = a.A[hh];
  const size_t tb0 = (size_t)b * T * H + hh;
  // first-token terms each unit handed to the next
  for (int u = tid; u + 1 < nu; u += blockDim.x) {
    const size_t t = (size_t)(u + 1) * Qu;
    a.ddt[tb0 + t * H] += ws.nxt[((size_t)chain * nu + u) * 2];
    a.dlam[tb0 + t * H] += ws.nxt[((size_t)chain * nu + u) * 2 + 1];
  }
  // the entry value E_0 = alpha_0 h0 + beta_0 sum_r x_prev (x) B_prev
  const float dt0 = a.dt[tb0], lm0 = a.lam[tb0];
  const float al0 = expf(dt0 * Ah);
  const float be0 = input_weights(dt0, lm0, al0, a.disc).x;
  const float* dE = ws.dE0 + (size_t)chain * PN;
  const float* h0 = a.h + (size_t)chain * PN;
  const IO* Bp0 = static_cast<const IO*>(a.B_prev) + (size_t)chain * R * N;
  const IO* Xp0 = static_cast<const IO*>(a.x_prev) + (size_t)chain * R * P;
  float dh_part = 0.f, du_part = 0.f;
  for (int e = tid; e < PN; e += blockDim.x) {
    const int p = e / N, n = e - p * N;
    const float gv = dE[e];
    a.dh0[(size_t)chain * PN + e] = al0 * gv;
    dh_part += gv * h0[e];
    float uv = 0.f;
    for (int r = 0; r < R; ++r) uv += to_f32(Xp0[r * P + p]) * to_f32(Bp0[r * N + n]);
    du_part += gv * uv;
  }
  const float sh = block_sum(dh_part, red);
  const float su = block_sum(du_part, red);
  for (int e = tid; e < R * P; e += blockDim.x) {  // dx_prev[r][p] = beta_0 sum_n dE[p][n] B_prev[r][n]
    const int r = e / P, p = e - r * P;
    float v = 0.f;
    for (int n = 0; n < N; ++n) v += dE[p * N + n] * to_f32(Bp0[r * N + n]);
    a.dx_prev[(size_t)chain * R * P + e] = be0 * v;
  }
  for (int e = tid; e < R * N; e += blockDim.x) {  // dB_prev[r][n] = beta_0 sum_p dE[p][n] x_prev[r][p]
    const int r = e / N, n = e - r * N;
    float v = 0.f;
    for (int p = 0; p < P; ++p) v += dE[p * N + n] * to_f32(Xp0[r * P + p]);
    a.dB_prev[(size_t)chain * R * N + e] = be0 * v;
  }
  if (tid == 0) {
    float dA = 0.f, dD = 0.f;
    for (int u = 0; u < nu; ++u) {
      dA += ws.upart[((size_t)chain * nu + u) * 2];
      dD += ws.upart[((size_t)chain * nu + u) * 2 + 1];
    }
    const DCoef dcf = dcoef(dt0, lm0, Ah, a.disc);
    const float da0 = al0 * sh;
    a.ddt[tb0] += Ah * da0 + dcf.bdt * su;
    a.dlam[tb0] += dcf.blam * su;
    ws.part[(size_t)chain * 2] = dA + dt0 * da0 + dcf.bA * su;
    ws.part[(size_t)chain * 2 + 1] = dD;
  }
}

// The unit kernels of one (P / 16, N / 16), then scan and finish.
// The local and grad kernels are compiled per rank (1, 2, 4: RS = 0, 1, 2),
// so their row -> (token, rank) arithmetic folds away.
template <typename IO, int PB, int NB, int RS>
hipError_t launch_io_pnr(const Dims& d, const BackwardArgs& a, const BwdWs& w, hipStream_t s) {
  constexpr int P = 16 * PB, N = 16 * NB;
  static bool attr_set = false;
  if (!attr_set) {
    const void* local;
    if constexpr (sizeof(IO) == 2)
      local = reinterpret_cast<const void*>(&local_bf_kernel<PB, NB, RS>);
    else
      local = reinterpret_cast<const void*>(&local_kernel<IO, PB, NB, RS>);
    for (const void* f : {local, reinterpret_cast<const void*>(&grad_kernel<IO, PB, NB, RS>)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  const int chains = d.batch * d.heads;
  const int nu = (a.seqlen + kU / d.R - 1) / (kU / d.R);
  const int bpc = (P * N / 8 + kScanT - 1) / kScanT;
  const size_t lds_local = (size_t)(kU * (P + 4) + kU * (N + 4) + (kU / d.R) * (N / 2 + 1) + kSmall) * 4;
  const size_t lds_grad = (size_t)Lay(P, N, d.R, true).total * 4;
  const dim3 units((unsigned)chains * nu), blk(kBT);
  if constexpr (sizeof(IO) == 2) {
    const size_t lds_bf = (size_t)(P + 3 * N) * 128 + (size_t)((kU / d.R) * (N / 2 + 1) + kSmall) * 4;
    hipLaunchKernelGGL((local_bf_kernel<PB, NB, RS>), dim3(2 * units.x), blk, lds_bf, s, a, w, d.heads, nu);
  } else {
    hipLaunchKernelGGL((local_kernel<IO, PB, NB, RS>), dim3(2 * units.x), blk, lds_local, s, a, w, d.heads, nu);
  }
  hipLaunchKernelGGL(scan_kernel<IO>, dim3(chains * bpc), dim3(kScanT), 0, s, a, w, d.heads, P, N, d.R, nu, bpc);
  hipLaunchKernelGGL((grad_kernel<IO, PB, NB, RS>), units, blk, lds_grad, s, a, w, d.heads, nu);
  hipLaunchKernelGGL(finish_kernel<IO>, dim3(chains), dim3(256), 0, s, a, w, d.heads, P, N, d.R, nu);
  return hipGetLastError();
}

template <typename IO, int PB, int NB>
hipError_t launch_io_pn(const Dims& d, const BackwardArgs& a, const BwdWs& w, hipStream_t s) {
  switch (d.R) {  // (the host accepts ranks 1, 2 and 4 only)
    case 1: return launch_io_pnr<IO, PB, NB, 0>(d, a, w, s);
    case 2: return launch_io_pnr<IO, PB, NB, 1>(d, a, w, s);
    case 4: return launch_io_pnr<IO, PB, NB, 2>(d, a, w, s);
    default: return hipErrorInvalidValue;
  }
}

// Dispatch over the supported tile counts (P, N in {16, 32, 64, 128}, P N <= 8192).
template <typename IO>
hipError_t launch_io(const Dims& d, const BackwardArgs& a, const BwdWs& w, hipStream_t s) {
#define M3_BWD_CASE(pb, nb) \
  if (d.P == 16 * pb && d.N == 16 * nb) return launch_io_pn<IO, pb, nb>(d, a, w, s);
  M3_BWD_CASE(1, 1) M3_BWD_CASE(1, 2) M3_BWD_CASE(1, 4) M3_BWD_CASE(1, 8)
  M3_BWD_CASE(2, 1) M3_BWD_CASE(2, 2) M3_BWD_CASE(2, 4) M3_BWD_CASE(2, 8)
  M3_BWD_CASE(4, 1) M3_BWD_CASE(4, 2) M3_BWD_CASE(4, 4) M3_BWD_CASE(4, 8)
  M3_BWD_CASE(8, 1) M3_BWD_CASE(8, 2) M3_BWD_CASE(8, 4)
#undef M3_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace bwd
}  // namespace m3
