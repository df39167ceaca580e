// Backward pass of the Mamba-3 scan for gfx950: gradients of
//     L = sum_t <dy_t, y_t> + <dh_final, h_T>
// with respect to every input of a prefill (lilting.ch Mamba-3 article,
// "アーキテクチャ改善" 1-3: exponential-trapezoid update, rotating state,
// rank-R coupling; the pages train these layers end to end but print no
// backward pass, so it is the exact derivative of the forward definition).
//
// One workgroup per chain (b, h).  The sequence is cut into sub-chunks of
// kRows / R tokens (16 (token, rank) rows).  Within a sub-chunk, in its own
// frame (angles phi_t and log-decays l_t counted from its first token, B and
// C rotated back by phi_t), the forward step is the masked dual form
//     Y   = (S . M) X + diag(e^l) Ct E^T + D X,        S = Ct Bt^T
//     E'  = Rot(phi_end) [ e^{l_E} E + sum_k w_k X_k (x) Bt_k ]
// with E the sub-chunk's entry value (the first token's decay and pending
// term applied), M the trapezoid mask, w the state-update weights (the next
// token's decay and previous-input weight folded in).  The kernel first runs
// the state recurrence forward over the sub-chunks and keeps every entry
// value E (and h_T) in the workspace; it then walks the sub-chunks in
// reverse, carrying the adjoint of E, and forms every gradient of the dual
// form: the row matrices (dX, dBt, dCt) and the adjoint of E from small
// contractions in LDS, the per-token scalars (mask, weights, decays) in one
// wave, and the rotations' angle gradients from the rotated rows.  The first
// token of a sub-chunk receives its decay and previous-input gradients from
// the sub-chunk before it (its alpha and beta live in that one's weights), so
// those two are added to the already written values.
//
// Arithmetic is fp32 throughout (VALU and LDS); gradients are written in fp32.
#include "m3_device.hpp"
#include "m3_kernels.hpp"

namespace m3 {
namespace {

constexpr int kBwdThreads = 512;
constexpr int kRows = 16;  // (token, rank) rows per sub-chunk

struct BwdLds {
  // floats
  static size_t bytes(int P, int N) {
    const size_t pn = (size_t)P * N;
    return 4 * (2 * pn + P               // E, G (then dE; rows padded by one)
                + (size_t)kRows * P * 3 + kRows  // X (padded), dY, G Bt
                + (size_t)kRows * N * 5 + kRows  // Bt (padded), Ct, dBt, dCt, carried part of dCt
                + 4 * kRows * kRows      // S, Pm, M, dM
                + (size_t)kRows * (N / 2) * 2  // phi, dphi
                + (N / 2)                // dphi_end
                + 16 * 16                // per-token scalars
                + 64);                   // reductions, misc
  }
};

// per-token scalar slots (sTk[slot * 16 + t])
enum { kA = 0, kAl, kBe, kGa, kL, kW, kEl, kDlc, kDw, kDt, kLm, kNumTk };

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = lane_group_sum(v, kWave);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < kBwdThreads / kWave; ++w) s += red[w];
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

template <typename IO>
__global__ __launch_bounds__(kBwdThreads) void backward_kernel(BackwardArgs a, int H, int P, int N, int R) {
  extern __shared__ __align__(16) float sm[];
  const int chain = blockIdx.x;
  const int hh = chain % H, b = chain / H;
  const int tid = threadIdx.x;
  const int T = a.seqlen;
  const int Qb = kRows / R;  // tokens per sub-chunk
  const int nsub = (T + Qb - 1) / Qb;
  const int NH = N / 2;
  const int PN = P * N;
  const float Ah = a.A[hh], Dh = a.D[hh];

  // rows of G, Bt and X are padded by one float: their column-wise reads (lanes
  // over p or over rows) then fall in distinct banks
  const int LDG = N + 1, LDB = N + 1, LDX = P + 1;
  float* sE = sm;
  float* sG = sE + PN;
  float* sX = sG + P * LDG;
  float* sdY = sX + kRows * LDX;
  float* sGB = sdY + kRows * P;
  float* sBt = sGB + kRows * P;
  float* sCt = sBt + kRows * LDB;
  float* sdBt = sCt + kRows * N;
  float* sdCt = sdBt + kRows * N;
  float* sCcar = sdCt + kRows * N;
  float* sS = sCcar + kRows * N;
  float* sPm = sS + kRows * kRows;
  float* sM = sPm + kRows * kRows;
  float* sdM = sM + kRows * kRows;
  float* sPhi = sdM + kRows * kRows;
  float* sDphi = sPhi + kRows * NH;
  float* sDphiE = sDphi + kRows * NH;
  float* sTk = sDphiE + NH;
  float* sMisc = sTk + 16 * 16;  // [0] lE, [1] a_next, [2] beta_next, [3] has_next, [8..] reductions

  const size_t tokBC = (size_t)H * R * N, tokX = (size_t)H * R * P, tokTh = (size_t)H * NH;
  const IO* Xg = static_cast<const IO*>(a.x) + ((size_t)b * T * H + hh) * R * P;
  const IO* Bg = static_cast<const IO*>(a.B) + ((size_t)b * T * H + hh) * R * N;
  const IO* Cg = static_cast<const IO*>(a.C) + ((size_t)b * T * H + hh) * R * N;
  const IO* dYg = static_cast<const IO*>(a.dy) + ((size_t)b * T * H + hh) * R * P;
  const float* DTg = a.dt + (size_t)b * T * H + hh;
  const float* LMg = a.lam + (size_t)b * T * H + hh;
  const float* THg = a.theta + ((size_t)b * T * H + hh) * NH;
  float* dXg = a.dx + ((size_t)b * T * H + hh) * R * P;
  float* dBg = a.dB + ((size_t)b * T * H + hh) * R * N;
  float* dCg = a.dC + ((size_t)b * T * H + hh) * R * N;
  float* dDTg = a.ddt + (size_t)b * T * H + hh;
  float* dLMg = a.dlam + (size_t)b * T * H + hh;
  float* dTHg = a.dtheta + ((size_t)b * T * H + hh) * NH;
  float* ck = a.ckpt + (size_t)chain * (nsub + 1) * PN;
  const IO* Bp0 = static_cast<const IO*>(a.B_prev) + (size_t)chain * R * N;
  const IO* Xp0 = static_cast<const IO*>(a.x_prev) + (size_t)chain * R * P;
  const float* h0 = a.h + (size_t)chain * PN;

  // P x N fp32 between the workspace and LDS in 16-byte runs, all loads of a
  // thread issued before their stores (a load per loop trip would wait for
  // each one in turn)
  constexpr int kMaxV = 8192 / 4 / kBwdThreads;  // float4s per thread at P N = 8192
  auto ld_state = [&](float* dst, const float* src) {
    float4 v[kMaxV];
#pragma unroll
    for (int i = 0; i < kMaxV; ++i) {  // clamped duplicates past the end, never stored
      const int e = tid + i * kBwdThreads;
      v[i] = reinterpret_cast<const float4*>(src)[e < PN / 4 ? e : PN / 4 - 1];
    }
#pragma unroll
    for (int i = 0; i < kMaxV; ++i) {
      const int e = tid + i * kBwdThreads;
      if (e < PN / 4) reinterpret_cast<float4*>(dst)[e] = v[i];
    }
  };
  auto st_state = [&](float* dst, const float* src) {
#pragma unroll
    for (int i = 0; i < kMaxV; ++i) {
      const int e = tid + i * kBwdThreads;
      if (e < PN / 4) reinterpret_cast<float4*>(dst)[e] = reinterpret_cast<const float4*>(src)[e];
    }
  };

  // ---- per-sub-chunk coefficients: token scalars, l, w, mask, angles ----
  // (wave 0, lane t = token: decays, weights; every thread: angle loads)
  auto coefs = [&](int c) {
    const int t0 = c * Qb, L = min(Qb, T - t0);
    const bool nxt = t0 + L < T;
    // the angles of the sub-chunk, all loads in flight together
    for (int e = tid; e < Qb * NH; e += kBwdThreads) {
      const int t = e / NH, j = e % NH;
      sPhi[e] = t < L ? THg[(size_t)(t0 + t) * tokTh + j] : 0.f;
    }
    if (tid < kWave) {
      const int t = tid;
      const bool v = t < L;
      // token t0 + L (the next one) in lane L: its decay and beta are folded in
      const bool vn = t == L && nxt;
      const int tg = t0 + (t < L ? t : L);
      const float dt = (v || vn) ? DTg[(size_t)tg * H] : 0.f;
      const float lm = (v || vn) ? LMg[(size_t)tg * H] : 0.f;
      const float al = expf(dt * Ah);
      const float2 bg = input_weights(dt, lm, al, a.disc);
      const float av = dt * Ah;
      // l_t = sum_{0<s<=t} a_s over the sub-chunk
      const float l = wave_inclusive_scan((v && t > 0) ? av : 0.f);
      const float lE = __shfl(l, L - 1, kWave) + __shfl(av, L, kWave);  // (lane L holds 0 without a next token)
      const float l_up = __shfl_down(l, 1, kWave);
      const float be_up = __shfl_down(bg.x, 1, kWave);
      if (v) {
        float w = bg.y * expf(lE - l);
        w += (t + 1 < L) ? be_up * expf(lE - l_up) : be_up;  // the next token's beta has weight e^{lE - lE}
        sTk[kA * 16 + t] = av;
        sTk[kDt * 16 + t] = dt;
        sTk[kLm * 16 + t] = lm;
        sTk[kAl * 16 + t] = al;
        sTk[kBe * 16 + t] = bg.x;
        sTk[kGa * 16 + t] = bg.y;
        sTk[kL * 16 + t] = l;
        sTk[kEl * 16 + t] = expf(l);
        sTk[kW * 16 + t] = w;
      }
      if (t == L) {
        sMisc[0] = lE;
        sMisc[1] = vn ? av : 0.f;
        sMisc[2] = vn ? bg.x : 0.f;
        sMisc[3] = vn ? 1.f : 0.f;
        sMisc[4] = dt;
        sMisc[5] = lm;
      }
    }
    __syncthreads();
    // inclusive angle prefix per pair; trapezoid mask over token pairs (q, k), k <= q
    for (int j = tid; j < NH; j += kBwdThreads) {
      float acc = 0.f;
      for (int t = 0; t < L; ++t) {
        acc += sPhi[t * NH + j];
        sPhi[t * NH + j] = acc;
      }
    }
    for (int e = tid; e < Qb * Qb; e += kBwdThreads) {
      const int q = e / Qb, k = e % Qb;
      float m = 0.f;
      if (q < L && k <= q) {
        const float lq = sTk[kL * 16 + q];
        m = sTk[kGa * 16 + k] * expf(lq - sTk[kL * 16 + k]);
        if (k < q) m += sTk[kBe * 16 + k + 1] * expf(lq - sTk[kL * 16 + k + 1]);
      }
      sM[e] = m;
    }
  };
  // ---- rows of x, rotated B (and C, dy) of sub-chunk c into LDS ----
  auto load_rows = [&](int c, bool with_c) {
    const int t0 = c * Qb, L = min(Qb, T - t0);
    const int nr = L * R;
    for (int e = tid; e < kRows * P; e += kBwdThreads) {
      const int rho = e / P, p = e % P;
      const bool ok = rho < nr;
      const size_t o = (size_t)(t0 + rho / R) * tokX + (rho % R) * P + p;
      sX[rho * LDX + p] = ok ? to_f32(Xg[o]) : 0.f;
      if (with_c) sdY[e] = ok ? to_f32(dYg[o]) : 0.f;
    }
    for (int e = tid; e < kRows * NH; e += kBwdThreads) {
      const int rho = e / NH, j = e % NH;
      float b0 = 0.f, b1 = 0.f, c0 = 0.f, c1 = 0.f;
      if (rho < nr) {
        const int t = rho / R;
        const size_t o = (size_t)(t0 + t) * tokBC + (rho % R) * N + 2 * j;
        float sn, cs;
        sincosf(sPhi[t * NH + j], &sn, &cs);
        const float v0 = to_f32(Bg[o]), v1 = to_f32(Bg[o + 1]);
        b0 = v0 * cs + v1 * sn;  // Rot(-phi)
        b1 = -v0 * sn + v1 * cs;
        if (with_c) {
          const float u0 = to_f32(Cg[o]), u1 = to_f32(Cg[o + 1]);
          c0 = u0 * cs + u1 * sn;
          c1 = -u0 * sn + u1 * cs;
        }
      }
      sBt[rho * LDB + 2 * j] = b0;
      sBt[rho * LDB + 2 * j + 1] = b1;
      if (with_c) {
        sCt[rho * N + 2 * j] = c0;
        sCt[rho * N + 2 * j + 1] = c1;
      }
    }
  };

  // ================= forward sweep: entry values of every sub-chunk =================
  // E_0 = alpha_0 h0 + beta_0 sum_r x_prev (x) B_prev
  {
    const float dt0 = DTg[0], lm0 = LMg[0];
    const float al0 = expf(dt0 * Ah);
    const float be0 = input_weights(dt0, lm0, al0, a.disc).x;
    for (int e = tid; e < PN; e += kBwdThreads) {
      const int p = e / N, n = e % N;
      float u = 0.f;
      for (int r = 0; r < R; ++r) u += to_f32(Xp0[r * P + p]) * to_f32(Bp0[r * N + n]);
      sE[e] = al0 * h0[e] + be0 * u;
    }
  }
  for (int c = 0; c < nsub; ++c) {
    coefs(c);
    load_rows(c, false);
    __syncthreads();
    st_state(ck + (size_t)c * PN, sE);
    const int L = min(Qb, T - c * Qb);
    const float elE = expf(sMisc[0]);
    // checkpoint, then E <- Rot(phi_end) [e^{lE} E + sum_rows w X (x) Bt]
    for (int e = tid; e < PN / 2; e += kBwdThreads) {
      const int p = e / NH, j = e % NH;
      const int i0 = p * N + 2 * j;
      float h0v = sE[i0], h1v = sE[i0 + 1];
      h0v *= elE;
      h1v *= elE;
      for (int rho = 0; rho < L * R; ++rho) {
        const float wx = sTk[kW * 16 + rho / R] * sX[rho * LDX + p];
        h0v += wx * sBt[rho * LDB + 2 * j];
        h1v += wx * sBt[rho * LDB + 2 * j + 1];
      }
      float sn, cs;
      sincosf(sPhi[(L - 1) * NH + j], &sn, &cs);
      sE[i0] = h0v * cs - h1v * sn;
      sE[i0 + 1] = h0v * sn + h1v * cs;
    }
    __syncthreads();
  }
  // sE keeps h_T (the successor entry value of the last sub-chunk); dE <- dh_final
  for (int e = tid; e < PN; e += kBwdThreads)
    sG[(e / N) * LDG + e % N] = a.dh_final ? a.dh_final[(size_t)chain * PN + e] : 0.f;
  __syncthreads();

  // ================= reverse sweep =================
  float* red = sMisc + 8;
  float dD_acc = 0.f, dA_acc = 0.f;  // thread 0 keeps the chain's dA; every thread its dD share
  // thread 0: gradients of a sub-chunk's first token stay pending until the
  // sub-chunk before it (walked next) has added its share
  float pend_ddt = 0.f, pend_dlam = 0.f;
  for (int c = nsub - 1; c >= 0; --c) {
    const int t0 = c * Qb, L = min(Qb, T - t0);
    const int nr = L * R;
    coefs(c);
    load_rows(c, true);
    __syncthreads();
    // G = Rot(-phi_end) dE_next, and the end angle's gradient
    // dphi_end[j] = sum_p (dE1 E'0 - dE0 E'1) with E' the next entry value
    // (still in sE: the previous step's entry value, or h_T)
    for (int j = tid; j < NH; j += kBwdThreads) {
      float sn, cs;
      sincosf(sPhi[(L - 1) * NH + j], &sn, &cs);
      float acc = 0.f;
      for (int p = 0; p < P; ++p) {
        const int i0 = p * N + 2 * j, ig = p * LDG + 2 * j;
        const float d0 = sG[ig], d1 = sG[ig + 1];
        acc += d1 * sE[i0] - d0 * sE[i0 + 1];
        sG[ig] = d0 * cs + d1 * sn;
        sG[ig + 1] = -d0 * sn + d1 * cs;
      }
      sDphiE[j] = acc;
    }
    __syncthreads();
    ld_state(sE, ck + (size_t)c * PN);
    __syncthreads();
    // scores S = Ct Bt^T, Pm = dY X^T (rows x rows)
    for (int e = tid; e < kRows * kRows; e += kBwdThreads) {
      const int q = e / kRows, k = e % kRows;
      float s = 0.f, pm = 0.f;
      if (q < nr && k < nr) {
        for (int n = 0; n < N; ++n) s += sCt[q * N + n] * sBt[k * LDB + n];
        for (int p = 0; p < P; ++p) pm += sdY[q * P + p] * sX[k * LDX + p];
      }
      sS[e] = s;
      sPm[e] = pm;
    }
    __syncthreads();
    // dM over token pairs (sum over the rank rows); dS = M Pm
    for (int e = tid; e < Qb * Qb; e += kBwdThreads) {
      const int tq = e / Qb, tk = e % Qb;
      float d = 0.f;
      for (int r = 0; r < R; ++r)
        for (int r2 = 0; r2 < R; ++r2) {
          const int i = (tq * R + r) * kRows + tk * R + r2;
          d += sS[i] * sPm[i];
        }
      sdM[e] = d;
    }
    // dX = (M.S)^T dY + D dY + w (G Bt);  G Bt kept for dw
    for (int e = tid; e < kRows * P; e += kBwdThreads) {
      const int k = e / P, p = e % P;
      float gb = 0.f, v = 0.f;
      if (k < nr) {
        for (int n = 0; n < N; ++n) gb += sG[p * LDG + n] * sBt[k * LDB + n];
        const int tk = k / R;
        for (int q = 0; q < nr; ++q) v += sM[(q / R) * Qb + tk] * sS[q * kRows + k] * sdY[q * P + p];
        v += Dh * sdY[e] + sTk[kW * 16 + tk] * gb;
        dXg[(size_t)(t0 + tk) * tokX + (k % R) * P + p] = v;
      }
      sGB[e] = gb;
    }
    // dCt = (M.Pm) Bt + e^l (E^T dY);  dBt = (M.Pm)^T Ct + w (G^T X)
    for (int e = tid; e < kRows * N; e += kBwdThreads) {
      const int q = e / N, n = e % N;
      float dc = 0.f, car = 0.f, db = 0.f;
      if (q < nr) {
        const int tq = q / R;
        for (int k = 0; k < nr; ++k) {
          const float mq = sM[tq * Qb + k / R];
          dc += mq * sPm[q * kRows + k] * sBt[k * LDB + n];
          const float mk = sM[(k / R) * Qb + tq];
          db += mk * sPm[k * kRows + q] * sCt[k * N + n];
        }
        float ed = 0.f, gx = 0.f;
        for (int p = 0; p < P; ++p) {
          ed += sE[p * N + n] * sdY[q * P + p];
          gx += sG[p * LDG + n] * sX[q * LDX + p];
        }
        car = sTk[kEl * 16 + tq] * ed;
        dc += car;
        db += sTk[kW * 16 + tq] * gx;
      }
      sdCt[e] = dc;
      sCcar[e] = car;
      sdBt[e] = db;
    }
    // <G, E> (the end decay's gradient) and <dY, X> (D's)
    float ge = 0.f, yx = 0.f;
    for (int e = tid; e < PN; e += kBwdThreads) ge += sG[(e / N) * LDG + e % N] * sE[e];
    for (int e = tid; e < kRows * P; e += kBwdThreads) yx += sdY[e] * sX[(e / P) * LDX + e % P];
    const float sumGE = block_sum(ge, red);
    dD_acc += yx;
    __syncthreads();
    // dE = e^{lE} G + sum_rows e^l dY (x) Ct   (in place: G is no longer read)
    {
      const float elE = expf(sMisc[0]);
      for (int e = tid; e < PN; e += kBwdThreads) {
        const int p = e / N, n = e % N;
        float v = elE * sG[p * LDG + n];
        for (int q = 0; q < nr; ++q) v += sTk[kEl * 16 + q / R] * sdY[q * P + p] * sCt[q * N + n];
        sG[p * LDG + n] = v;
      }
    }
    // rows back to the lab frame (dB, dC), angle gradients per (token, pair)
    for (int e = tid; e < kRows * NH; e += kBwdThreads) {
      const int q = e / NH, j = e % NH;
      if (q < nr) {
        const int t = q / R;
        float sn, cs;
        sincosf(sPhi[t * NH + j], &sn, &cs);
        const float db0 = sdBt[q * N + 2 * j], db1 = sdBt[q * N + 2 * j + 1];
        const float dc0 = sdCt[q * N + 2 * j], dc1 = sdCt[q * N + 2 * j + 1];
        const size_t o = (size_t)(t0 + t) * tokBC + (q % R) * N + 2 * j;
        dBg[o] = db0 * cs - db1 * sn;  // Rot(+phi)
        dBg[o + 1] = db0 * sn + db1 * cs;
        dCg[o] = dc0 * cs - dc1 * sn;
        dCg[o + 1] = dc0 * sn + dc1 * cs;
      }
    }
    for (int e = tid; e < Qb * NH; e += kBwdThreads) {
      const int t = e / NH, j = e % NH;
      float d = 0.f;
      if (t < L) {
        for (int r = 0; r < R; ++r) {
          const int q = t * R + r;
          d += sdBt[q * N + 2 * j] * sBt[q * LDB + 2 * j + 1] - sdBt[q * N + 2 * j + 1] * sBt[q * LDB + 2 * j];
          d += sdCt[q * N + 2 * j] * sCt[q * N + 2 * j + 1] - sdCt[q * N + 2 * j + 1] * sCt[q * N + 2 * j];
        }
      }
      sDphi[e] = d;
    }
    // per-token reductions: carried decay gradient and state-update weight gradient
    for (int t = tid / kWave; t < L; t += kBwdThreads / kWave) {
      const int lane = tid % kWave;
      float dlc = 0.f, dw = 0.f;
      for (int r = 0; r < R; ++r) {
        const int q = t * R + r;
        for (int n = lane; n < N; n += kWave) dlc += sCcar[q * N + n] * sCt[q * N + n];
        for (int p = lane; p < P; p += kWave) dw += sX[q * LDX + p] * sGB[q * P + p];
      }
      dlc = lane_group_sum(dlc, kWave);
      dw = lane_group_sum(dw, kWave);
      if (lane == 0) {
        sTk[kDlc * 16 + t] = dlc;
        sTk[kDw * 16 + t] = dw;
      }
    }
    __syncthreads();
    // angles: dtheta_s = sum_{t >= s} dphi_t + dphi_end
    for (int j = tid; j < NH; j += kBwdThreads) {
      float acc = sDphiE[j];
      for (int t = L - 1; t >= 0; --t) {
        acc += sDphi[t * NH + j];
        dTHg[(size_t)(t0 + t) * tokTh + j] = acc;
      }
    }
    // token scalars, lane t of wave 0 = token t.  With the pairs' and the
    // weights' terms collected per token,
    //   dgamma_t = sum_{q>=t} dM(q,t) e^{l_q-l_t} + dw_t e^{lE-l_t}
    //   dbeta_t  = sum_{q>=t} dM(q,t-1) e^{l_q-l_t} + dw_{t-1} e^{lE-l_t}   (t >= 1)
    //   dl_t     = (carried part) + sum_{k<=t} dM(t,k) M(t,k) - gamma_t dgamma_t - beta_t dbeta_t
    //   dlE      = e^{lE} <G, E> + sum_k dw_k (w_k - [k = L-1] beta_next)
    // and the log-decays' sums l_t = sum_{0<s<=t} a_s, lE = l_{L-1} + a_next.
    if (tid < kWave) {
      const int t = tid;
      const bool v = t < L;
      const float lE = sMisc[0];
      const bool nxt = sMisc[3] != 0.f;
      float dga = 0.f, dbe = 0.f, dl = 0.f, dwt = 0.f, wpart = 0.f;
      if (v) {
        const float lt = sTk[kL * 16 + t];
        dwt = sTk[kDw * 16 + t];
        for (int q = t; q < L; ++q) {
          const float e = expf(sTk[kL * 16 + q] - lt);
          dga += sdM[q * Qb + t] * e;
          if (t >= 1) dbe += sdM[q * Qb + t - 1] * e;
        }
        dga += dwt * expf(lE - lt);
        if (t >= 1) dbe += sTk[kDw * 16 + t - 1] * expf(lE - lt);
        float dlq = sTk[kDlc * 16 + t];
        for (int k = 0; k <= t; ++k) dlq += sdM[t * Qb + k] * sM[t * Qb + k];
        dl = dlq - sTk[kGa * 16 + t] * dga - (t >= 1 ? sTk[kBe * 16 + t] * dbe : 0.f);
        wpart = dwt * (sTk[kW * 16 + t] - (t == L - 1 ? sMisc[2] : 0.f));
      }
      const float dlE = expf(lE) * sumGE + lane_group_sum(wpart, kWave);
      const float dbn = __shfl(dwt, L - 1, kWave);  // beta of the next token, weight e^{lE - lE} = 1
      const float pre = wave_inclusive_scan(dl);
      const float rc = lane_group_sum(dl, kWave) - pre + dl;  // sum_{s >= t} dl_s
      float gdt = 0.f, glm = 0.f, dAp = 0.f;
      if (v) {
        const float da = t > 0 ? rc + dlE : 0.f;
        const float dt = sTk[kDt * 16 + t], lm = sTk[kLm * 16 + t];
        const DCoef dc = dcoef(dt, lm, Ah, a.disc);
        gdt = Ah * da + dc.bdt * dbe + dc.gdt * dga;
        glm = dc.blam * dbe + dc.glam * dga;
        dAp = dt * da + dc.bA * dbe;
        if (t > 0) {
          dDTg[(size_t)(t0 + t) * H] = gdt;
          dLMg[(size_t)(t0 + t) * H] = glm;
        }
      }
      dAp = lane_group_sum(dAp, kWave);
      if (t == 0) {
        if (nxt) {  // the next token's decay and previous-input weight entered here
          const float dt = sMisc[4], lm = sMisc[5];
          const DCoef dc = dcoef(dt, lm, Ah, a.disc);
          dDTg[(size_t)(t0 + L) * H] = pend_ddt + Ah * dlE + dc.bdt * dbn;
          dLMg[(size_t)(t0 + L) * H] = pend_dlam + dc.blam * dbn;
          dA_acc += dt * dlE + dc.bA * dbn;
        }
        pend_ddt = gdt;
        pend_dlam = glm;
        dA_acc += dAp;
      }
    }
    __syncthreads();
  }
  // ================= the entry: E_0 = alpha_0 h0 + beta_0 u_prev =================
  {
    const float dt0 = DTg[0], lm0 = LMg[0];
    const float al0 = expf(dt0 * Ah);
    const float be0 = input_weights(dt0, lm0, al0, a.disc).x;
    float dh_part = 0.f, du_part = 0.f;
    for (int e = tid; e < PN; e += kBwdThreads) {
      const int p = e / N, n = e % N;
      const float g = sG[p * LDG + n];
      a.dh0[(size_t)chain * PN + e] = al0 * g;
      dh_part += g * h0[e];
      float u = 0.f;
      for (int r = 0; r < R; ++r) u += to_f32(Xp0[r * P + p]) * to_f32(Bp0[r * N + n]);
      du_part += g * u;
    }
    const float sh = block_sum(dh_part, red);
    const float su = block_sum(du_part, red);
    for (int e = tid; e < R * P; e += kBwdThreads) {  // dx_prev[r][p] = beta_0 sum_n dE[p][n] B_prev[r][n]
      const int r = e / P, p = e % P;
      float v = 0.f;
      for (int n = 0; n < N; ++n) v += sG[p * LDG + n] * to_f32(Bp0[r * N + n]);
      a.dx_prev[(size_t)chain * R * P + e] = be0 * v;
    }
    for (int e = tid; e < R * N; e += kBwdThreads) {  // dB_prev[r][n] = beta_0 sum_p dE[p][n] x_prev[r][p]
      const int r = e / N, n = e % N;
      float v = 0.f;
      for (int p = 0; p < P; ++p) v += sG[p * LDG + n] * to_f32(Xp0[r * P + p]);
      a.dB_prev[(size_t)chain * R * N + e] = be0 * v;
    }
    const float dsum = block_sum(dD_acc, red);
    if (tid == 0) {
      const DCoef dc = dcoef(dt0, lm0, Ah, a.disc);
      const float da0 = al0 * sh;
      a.ddt[(size_t)b * T * H + hh] = pend_ddt + Ah * da0 + dc.bdt * su;
      a.dlam[(size_t)b * T * H + hh] = pend_dlam + dc.blam * su;
      dA_acc += dt0 * da0 + dc.bA * su;
      a.part[(size_t)chain * 2] = dA_acc;
      a.part[(size_t)chain * 2 + 1] = dsum;
    }
  }
}

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

}  // namespace

bool backward_supported(const Dims& d) {
  return (d.R == 1 || d.R == 2 || d.R == 4) && d.N >= 2 && d.N % 2 == 0 && d.N <= 128 && d.P <= 128 &&
         d.P * d.N <= 8192 && BwdLds::bytes(d.P, d.N) <= 160 * 1024;
}

size_t backward_workspace_bytes(const Dims& d, int seqlen) {
  const int Qb = kRows / d.R;
  const size_t nsub = (size_t)(seqlen + Qb - 1) / Qb;
  const size_t chains = (size_t)d.batch * d.heads;
  return chains * (nsub + 1) * d.P * d.N * 4 + ((chains * 2 * 4 + 255) & ~(size_t)255);
}

hipError_t launch_backward(const Dims& d, const BackwardArgs& a, hipStream_t s) {
  const size_t lds = BwdLds::bytes(d.P, d.N);
  static bool attr_set = false;
  if (!attr_set) {
    for (const void* f : {reinterpret_cast<const void*>(&backward_kernel<bf16>),
                          reinterpret_cast<const void*>(&backward_kernel<float>)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  const dim3 grid(d.batch * d.heads), block(kBwdThreads);
  if (d.bf16)
    hipLaunchKernelGGL(backward_kernel<bf16>, grid, block, lds, s, a, d.heads, d.P, d.N, d.R);
  else
    hipLaunchKernelGGL(backward_kernel<float>, grid, block, lds, s, a, d.heads, d.P, d.N, d.R);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(backward_reduce_kernel, dim3((d.heads + 63) / 64), dim3(64), 0, s, a.part, a.dA, a.dD, d.batch,
                     d.heads);
  return hipGetLastError();
}

}  // namespace m3
