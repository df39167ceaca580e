// Mamba-3 chunked prefill for gfx950.
//
// Method (lilting.ch Mamba-3 article, "アーキテクチャ改善" 1-3; the chunked
// "dual" form is the matmul-shaped restructuring the article's SSM-history
// section credits to Mamba-2):  per (batch, head) chain, tokens are processed
// in chunks of Q.  Inside a chunk starting at c0, with local frame angles
// phi_t = sum_{k=c0..t} theta_k and rotated operands
//     Bt_s = Rot(-phi_s) B_s,   Ct_t = Rot(-phi_t) C_t,
// the state in the local frame is
//     g_t = e^{l_t} E + sum_{s<=t} M[t,s] x_s (x) Bt_s,      l_t = sum_{k=c0+1..t} dt_k A,
//     M[t,s] = gamma_s e^{l_t - l_s} + [s<t] beta_{s+1} e^{l_t - l_{s+1}},
// where E = alpha_{c0} h_{c0-1} + beta_{c0} x_{c0-1} (x) B_{c0-1} is the
// "entry value" of the chunk: the carried lab-frame state with the first
// token's decay and its previous-input term already applied.  Then
//     y_t = e^{l_t} Ct_t E  +  sum_{s<=t} M[t,s] (Ct_t . Bt_s) x_s  +  D x_t
// and the next chunk's entry value is
//     E' = Rot(phi_e) [ e^{l_E} E + sum_s w_s x_s (x) Bt_s ],
//     l_E = l_e + dt_{e+1} A,  w_s = gamma_s e^{l_E - l_s} + beta_{s+1} e^{l_E - l_{s+1}}
// (beta_{e+1}, dt_{e+1} belong to the first token of the next chunk; both are
// 0 after the last token, which makes E' the final lab-frame state h_T).
// Folding the next token's coefficients into E removes the separate
// "previous token" key that the trapezoid rule would otherwise add to every
// chunk.  MIMO rank R: rows and keys are (token, rank) pairs; M depends on the
// tokens only, and the R ranks share the state.
//
// gfx950 mapping.  One workgroup of 4 waves walks one chain (or one segment of
// a chain) chunk by chunk; the P x N fp32 state never leaves registers.  Per
// chunk:
//   A1  wave 0: in-chunk log-decay scan (one wave64 prefix scan), per-token
//       mask coefficients -> LDS.
//   A2  angle prefix over the chunk per state pair, 4 tokens per thread plus
//       a cross-group pass through LDS.
//   A3  16-byte coalesced loads of B, C, x; rotation by -phi; bf16/fp32 tiles
//       to LDS: Bt and Ct row-major, Bt^T scaled by w (for the state update),
//       X^T (p-major).
//   B   per 16-row block (waves take row blocks in a balanced snake order):
//       S^T = Bt Ct^T on MFMA (16x16x32 bf16 or 16x16x4 f32), causal mask
//       applied in registers, the masked tile re-used directly as the A
//       operand of (S.M) X (the key order inside the 32-wide K slab is the
//       accumulator order, and X^T is read in the same order), plus
//       e^{l_t} Ct E from the bf16/fp32 copy of E in LDS, plus D x.
//   C   state update on MFMA: E^T tiles (rows n, cols p) += (Bt^T w) X, then
//       the pair rotation by phi_e, which is lane-local in that layout.
// Long prompts of few chains run in three passes (segment summaries from a
// zero entry value, a wave-level scan over segments, then every segment from
// its true entry value).
#include "m3_device.hpp"
#include "m3_kernels.hpp"
#include "m3_mfma.hpp"

namespace m3 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;

enum Mode : int { kFused = 0, kSummary = 1, kSegment = 2 };

// ----------------------------------------------------------------------------
// LDS layout (dynamic).  rows = Q*R rounded up to 32; all pitches add 16 B.
// ----------------------------------------------------------------------------
template <typename IO, int N, int P>
struct Lds {
  static constexpr int E = sizeof(IO);
  static constexpr int PAD = 16 / E;
  static constexpr int NK = N < 32 ? 32 : N;  // contraction width over N (zero-padded to a 32 slab)
  static constexpr int LDN = NK + PAD;        // pitch of sB, sC, sH rows (elements)
  int rows, ldr;                       // padded row count, pitch of sBt / sXt
  IO *sB, *sC, *sBt, *sXt, *sH;
  float* sPhi;   // [Q][N/2] chunk-local angles
  float* sTot;   // [Q/4][N/2] per-4-token angle totals
  float4* sTok;  // [Q] {gamma, l*log2e, beta_next, l_next*log2e}
  float* sW;     // [Q] state-update weights w_s
  float* sMisc;  // [0] l_E (natural log), [1] l_E*log2e
  float* sSeg;   // [N/2] running angle total (segment summaries)
  float2* sEnd;  // [N/2] (cos, sin) of the chunk's last local angle

  __host__ __device__ static constexpr size_t bytes(int rows_pad, int Q) {
    const int ldr = rows_pad + PAD;
    size_t b = 0;
    b += (size_t)rows_pad * LDN * E * 2;  // sB, sC
    b += (size_t)N * ldr * E;             // sBt
    b += (size_t)P * ldr * E;             // sXt
    b += (size_t)P * LDN * E;             // sH
    b += (size_t)Q * (N / 2) * 4;         // sPhi
    b += (size_t)(Q / 4) * (N / 2) * 4;   // sTot
    b += (size_t)Q * 16;                  // sTok
    b += (size_t)Q * 4;                   // sW
    b += 16;                              // sMisc
    b += (size_t)(N / 2) * 4;             // sSeg
    b += (size_t)(N / 2) * 8;             // sEnd
    return b;
  }
  __device__ void carve(char* base, int rows_pad, int Q) {
    rows = rows_pad;
    ldr = rows_pad + PAD;
    char* p = base;
    sB = reinterpret_cast<IO*>(p); p += (size_t)rows_pad * LDN * E;
    sC = reinterpret_cast<IO*>(p); p += (size_t)rows_pad * LDN * E;
    sBt = reinterpret_cast<IO*>(p); p += (size_t)N * ldr * E;
    sXt = reinterpret_cast<IO*>(p); p += (size_t)P * ldr * E;
    sH = reinterpret_cast<IO*>(p); p += (size_t)P * LDN * E;
    sPhi = reinterpret_cast<float*>(p); p += (size_t)Q * (N / 2) * 4;
    sTot = reinterpret_cast<float*>(p); p += (size_t)(Q / 4) * (N / 2) * 4;
    sTok = reinterpret_cast<float4*>(p); p += (size_t)Q * 16;
    sW = reinterpret_cast<float*>(p); p += (size_t)Q * 4;
    sMisc = reinterpret_cast<float*>(p); p += 16;
    sSeg = reinterpret_cast<float*>(p); p += (size_t)(N / 2) * 4;
    sEnd = reinterpret_cast<float2*>(p);
  }
};

// Largest padded row count (Q*R rounded up to 32) a <IO, N, P> instance
// supports: the LDS tiles must fit 160 KiB and every thread prefetches at
// most two 4-row x 8-column slices of B, C and x.
template <typename IO, int N, int P>
struct Limits {
  static constexpr size_t kLds = 160 * 1024;
  static constexpr bool fits(int r) {
    return Lds<IO, N, P>::bytes(r, r < 64 ? r : 64) <= kLds && r * N <= 16384 && r * P <= 16384;
  }
  static constexpr int kMaxRows = fits(256) ? 256 : fits(128) ? 128 : fits(64) ? 64 : fits(32) ? 32 : 0;
  static constexpr int kMaxB = (kMaxRows / 4) * (N / 8) > kThreads ? 2 : 1;  // B/C slices per thread
  static constexpr int kMaxX = (kMaxRows / 4) * (P / 8) > kThreads ? 2 : 1;  // x slices per thread
};

struct KParams {
  PrefillArgs a;
  int batch, heads, R, lgR, Q;
  int mode;
  int nblocks;  // grid size
};

// Workgroup -> (chain, segment).  Consecutive workgroups land on different
// XCDs (round-robin over 8); the remap puts consecutive chains -- the heads of
// one batch row, which share cache lines of dt and lam -- on the same XCD.
__device__ __forceinline__ int remap_block(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

template <typename IO, int N, int P>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(KParams kp) {
  using L = Lds<IO, N, P>;
  constexpr int NB = N / 16, PB = P / 16, NT = NB * PB;
  constexpr int TPW = (NT + kWaves - 1) / kWaves;  // state tiles per wave
  constexpr int NS = L::NK / 32;                    // 32-wide K slabs over N (padded)
  constexpr int LDN = L::LDN;
  extern __shared__ __align__(16) char smem[];

  const PrefillArgs& a = kp.a;
  const int Q = kp.Q, R = kp.R, lgR = kp.lgR, H = kp.heads;
  const int T = a.seqlen;
  const int mode = kp.mode;
  const int nseg_grid = (mode == kFused) ? 1 : (mode == kSummary ? a.nseg - 1 : a.nseg);
  const int bid = remap_block(blockIdx.x, kp.nblocks);
  const int chain = bid / nseg_grid;
  const int seg = bid % nseg_grid;
  const int b = chain / H, hh = chain % H;
  const int nchunks = (T + Q - 1) / Q;
  const int ck0 = (mode == kFused) ? 0 : seg * a.seg_chunks;
  int ck1 = (mode == kFused) ? nchunks : ck0 + a.seg_chunks;
  if (ck1 > nchunks) ck1 = nchunks;
  const bool writes_final = (mode == kFused) || (mode == kSegment && seg == a.nseg - 1);
  const bool has_y = mode != kSummary;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int rows = Q * R;
  const int rows_pad = (rows + 31) & ~31;
  L s;
  s.carve(smem, rows_pad, Q);
  const int ldr = s.ldr;
  if (L::NK != N) {
    // columns N .. NK-1 of sB, sC and sH are never written: keep them zero
    for (int e = tid; e < rows_pad * LDN; e += kThreads) {
      s.sB[e] = from_f32<IO>(0.f);
      s.sC[e] = from_f32<IO>(0.f);
    }
    for (int e = tid; e < P * LDN; e += kThreads) s.sH[e] = from_f32<IO>(0.f);
    __syncthreads();
  }

  const float Ah = a.A[hh];
  const float Dh = a.D[hh];
  // Strides (elements) of the (b, T, H, ...) layouts.
  const size_t tokBC = (size_t)H * R * N;  // B, C per token
  const size_t tokX = (size_t)H * R * P;   // x, y per token
  const size_t tokTh = (size_t)H * (N / 2);
  const IO* Bg = static_cast<const IO*>(a.B) + ((size_t)b * T * H + hh) * R * N;
  const IO* Cg = static_cast<const IO*>(a.C) + ((size_t)b * T * H + hh) * R * N;
  const IO* Xg = static_cast<const IO*>(a.x) + ((size_t)b * T * H + hh) * R * P;
  IO* Yg = static_cast<IO*>(a.y) + ((size_t)b * T * H + hh) * R * P;
  const float* THg = a.theta + ((size_t)b * T * H + hh) * (N / 2);
  const float* DTg = a.dt + (size_t)b * T * H + hh;
  const float* LMg = a.lam + (size_t)b * T * H + hh;

  // ---------------- entry value E of the first chunk ----------------
  f32x4 Hreg[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) Hreg[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    float alpha0 = 0.f, beta0 = 0.f;
    if (mode == kFused) {
      const float dt0 = DTg[(size_t)ck0 * Q * H];
      const float lm0 = LMg[(size_t)ck0 * Q * H];
      alpha0 = expf(dt0 * Ah);
      beta0 = input_weights(dt0, lm0, alpha0, a.disc).x;
    }
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int tile = wave + k * kWaves;
      if (tile < NT) {
        const int nb = tile / PB, pb = tile % PB;
        const int p = 16 * pb + c, n0 = 16 * nb + 4 * g;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (mode == kFused) {
          float h0[4];
          load4(a.h + ((size_t)chain * P + p) * N + n0, h0);
          const IO* Bp = static_cast<const IO*>(a.B_prev) + (size_t)chain * R * N;
          const IO* Xp = static_cast<const IO*>(a.x_prev) + (size_t)chain * R * P;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = alpha0 * h0[i];
          for (int r = 0; r < R; ++r) {
            float bp[4];
            load4(Bp + r * N + n0, bp);
            const float xp = beta0 * to_f32(Xp[r * P + p]);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] += xp * bp[i];
          }
        } else if (mode == kSegment) {
          load4(a.seg_state + (((size_t)seg * kp.batch * H + chain) * P + p) * N + n0, v);
        }
        Hreg[k] = f32x4{v[0], v[1], v[2], v[3]};
        store4(s.sH + p * LDN + n0, v);
      }
    }
  }
  if (mode == kSummary) {
    for (int j = tid; j < N / 2; j += kThreads) s.sSeg[j] = 0.f;
  }
  float lsum = 0.f;  // running log-decay of a segment summary (thread 0)

  // ---------------- register prefetch of one chunk's inputs ----------------
  // Issued for chunk c+1 right after chunk c's tiles are built, so the HBM
  // latency overlaps chunk c's matrix-core phases.
  constexpr int MB = Limits<IO, N, P>::kMaxB, MX = Limits<IO, N, P>::kMaxX;
  const int npg = N / 8;                        // pair groups of 4 pairs (8 columns)
  const int nth = (Q / 4) * npg;                // angle items (4 tokens x 4 pairs), <= 256
  const int nbitems = (rows_pad / 4) * npg;     // B/C items (4 rows x 8 columns)
  const int npx = P / 8;
  const int nxitems = (rows_pad / 4) * npx;     // x items (4 rows x 8 columns)
  float pf_dt = 0.f, pf_lm = 0.f, pf_dtn = 0.f, pf_lmn = 0.f;
  float4 pf_th[4];
  Raw8<IO> pf_b[MB][4], pf_c[MB][4], pf_x[MX][4];

  // Loads are unconditional from clamped (always valid) addresses; rows and
  // tokens past the end are zeroed where the values are consumed.  A load
  // into a register that was zeroed on another path would make the compiler
  // wait for every outstanding load before the next one.
  auto issue_loads = [&](int ck) {
    const int c0 = ck * Q;
    const int Lc = (T - c0 < Q) ? (T - c0) : Q;
    if (wave == 0) {
      const int t = lane < Lc ? lane : Lc - 1;
      pf_dt = DTg[(size_t)(c0 + t) * H];
      pf_lm = LMg[(size_t)(c0 + t) * H];
      const int tn = (c0 + Lc < T) ? c0 + Lc : c0 + Lc - 1;
      pf_dtn = DTg[(size_t)tn * H];
      pf_lmn = LMg[(size_t)tn * H];
    }
    if (tid < nth) {
      const int tg = tid / npg, pg = tid % npg;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = (4 * tg + k < Lc) ? 4 * tg + k : 0;
        pf_th[k] = *reinterpret_cast<const float4*>(THg + (size_t)(c0 + t) * tokTh + 4 * pg);
      }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int it = tid + m * kThreads;
      if (it < nbitems) {
        const int rg = it / npg, cg = it % npg;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int rho = 4 * rg + k;
          const bool valid = rho < rows && (rho >> lgR) < Lc;
          const int t = valid ? (rho >> lgR) : 0, r = valid ? (rho & (R - 1)) : 0;
          pf_b[m][k].load(Bg + (size_t)(c0 + t) * tokBC + r * N + 8 * cg);
          if (has_y) pf_c[m][k].load(Cg + (size_t)(c0 + t) * tokBC + r * N + 8 * cg);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MX; ++m) {
      const int it = tid + m * kThreads;
      if (it < nxitems) {
        const int rg = it / npx, xg = it % npx;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int rho = 4 * rg + k;
          const bool valid = rho < rows && (rho >> lgR) < Lc;
          const int t = valid ? (rho >> lgR) : 0, r = valid ? (rho & (R - 1)) : 0;
          pf_x[m][k].load(Xg + (size_t)(c0 + t) * tokX + r * P + 8 * xg);
        }
      }
    }
  };

  if (ck0 < ck1) issue_loads(ck0);

  for (int ck = ck0; ck < ck1; ++ck) {
    const int c0 = ck * Q;
    const int Lc = (T - c0 < Q) ? (T - c0) : Q;  // valid tokens in this chunk
    const bool fold_next = (c0 + Lc) < T;        // a token follows this chunk
    const int te = Lc - 1;
    __syncthreads();  // previous chunk fully consumed (LDS reuse)

    // ---------------- A1: decay scan and per-token coefficients ----------------
    if (wave == 0) {
      const int t = lane;
      const bool valid = t < Lc;
      const float dtv = valid ? pf_dt : 0.f, lmv = valid ? pf_lm : 0.f;
      const float av = (valid && t > 0) ? log_decay(dtv, Ah) : 0.f;
      const float ell = wave_inclusive_scan(av);   // l_t (first token's decay is in E)
      const float2 wt = input_weights(dtv, lmv, expf(dtv * Ah), a.disc);
      const float bet = wt.x, gam = wt.y;
      const float dtn = fold_next ? pf_dtn : 0.f;
      const float lmn = fold_next ? pf_lmn : 0.f;
      const float ell_last = __shfl(ell, Lc - 1, kWave);
      const float ellE = ell_last + log_decay(dtn, Ah);
      const float bet_next_tok = input_weights(dtn, lmn, expf(dtn * Ah), a.disc).x;
      const float bet_up = __shfl_down(bet, 1, kWave);
      const float ell_up = __shfl_down(ell, 1, kWave);
      float betn, elln;
      if (t < Lc - 1) {
        betn = bet_up;
        elln = ell_up;
      } else if (t == Lc - 1) {
        betn = bet_next_tok;
        elln = ellE;
      } else {
        betn = 0.f;
        elln = ellE;
      }
      const float ellv = valid ? ell : ell_last;
      const float w = valid ? (gam * expf(ellE - ellv) + betn * expf(ellE - elln)) : 0.f;
      if (t < Q) {
        s.sTok[t] = make_float4(valid ? gam : 0.f, ellv * kLog2e, valid ? betn : 0.f, elln * kLog2e);
        s.sW[t] = w;
      }
      if (t == 0) {
        s.sMisc[0] = ellE;
        s.sMisc[1] = ellE * kLog2e;
      }
      if (mode == kSummary && t == 0) lsum += ellE;
    }

    // ---------------- A2: angle prefix over the chunk ----------------
    float ph[4][4];
    const int tg = tid / npg, pg = tid % npg;
    if (tid < nth) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool tv = 4 * tg + k < Lc;
        ph[k][0] = tv ? reduce_angle(pf_th[k].x) : 0.f;
        ph[k][1] = tv ? reduce_angle(pf_th[k].y) : 0.f;
        ph[k][2] = tv ? reduce_angle(pf_th[k].z) : 0.f;
        ph[k][3] = tv ? reduce_angle(pf_th[k].w) : 0.f;
        if (k > 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) ph[k][j] += ph[k - 1][j];
        }
      }
      *reinterpret_cast<float4*>(s.sTot + tg * (N / 2) + 4 * pg) =
          make_float4(ph[3][0], ph[3][1], ph[3][2], ph[3][3]);
    }
    __syncthreads();
    if (tid < nth) {
      float off[4] = {0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < tg; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(s.sTot + q * (N / 2) + 4 * pg);
        off[0] += v.x; off[1] += v.y; off[2] += v.z; off[3] += v.w;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) ph[k][j] += off[j];
        *reinterpret_cast<float4*>(s.sPhi + (4 * tg + k) * (N / 2) + 4 * pg) =
            make_float4(ph[k][0], ph[k][1], ph[k][2], ph[k][3]);
        if (4 * tg + k == te) {
          // rotation of the carried state into the next chunk's frame (fp32 trig)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float sn, cs;
            sincosf(ph[k][j], &sn, &cs);
            s.sEnd[4 * pg + j] = make_float2(cs, sn);
          }
        }
      }
    }
    __syncthreads();

    // ---------------- A3: rotate B, C; build the LDS tiles ----------------
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int it = tid + m * kThreads;
      if (it < nbitems) {
        const int rg = it / npg, cg = it % npg;
        float bt[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int rho = 4 * rg + k;
          const int t = rho >> lgR;
          const bool valid = (rho < rows) && (t < Lc);
          float bv[8], cv[8];
          pf_b[m][k].unpack(bv);
          if (has_y) pf_c[m][k].unpack(cv);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            bv[e] = valid ? bv[e] : 0.f;
            cv[e] = (valid && has_y) ? cv[e] : 0.f;
          }
          float wt = 0.f;
          if (valid) {
            const float4 pv = *reinterpret_cast<const float4*>(s.sPhi + t * (N / 2) + 4 * cg);
            const float pa[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float sn, cs;
              trig<IO>(pa[j], sn, cs);
              // Rot(-phi): (u, v) -> (u c + v s, -u s + v c)
              rot2(bv[2 * j], bv[2 * j + 1], cs, -sn);
              rot2(cv[2 * j], cv[2 * j + 1], cs, -sn);
            }
            wt = s.sW[t];
          }
          store8(s.sB + rho * LDN + 8 * cg, bv);
          if (has_y) store8(s.sC + rho * LDN + 8 * cg, cv);
#pragma unroll
          for (int e = 0; e < 8; ++e) bt[k][e] = bv[e] * wt;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float col[4] = {bt[0][e], bt[1][e], bt[2][e], bt[3][e]};
          store4(s.sBt + (8 * cg + e) * ldr + 4 * rg, col);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MX; ++m) {
      const int it = tid + m * kThreads;
      if (it < nxitems) {
        const int rg = it / npx, xg = it % npx;
        float xv[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int rho = 4 * rg + k;
          const bool valid = rho < rows && (rho >> lgR) < Lc;
          pf_x[m][k].unpack(xv[k]);
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[k][e] = valid ? xv[k][e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float col[4] = {xv[0][e], xv[1][e], xv[2][e], xv[3][e]};
          store4(s.sXt + (8 * xg + e) * ldr + 4 * rg, col);
        }
      }
    }
    // next chunk's inputs: in flight during this chunk's matrix-core phases
    if (ck + 1 < ck1) issue_loads(ck + 1);
    __syncthreads();

    // ---------------- B: outputs of this chunk ----------------
    if (has_y) {
      const int nrb = (Lc * R + 15) / 16;  // row blocks holding valid rows
      for (int round = 0; round * kWaves < nrb; ++round) {
        const int rb = round * kWaves + ((round & 1) ? (kWaves - 1 - wave) : wave);
        if (rb >= nrb) continue;
        f32x4 Y[PB];
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) Y[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // carried-state term: Ct E, then the row scale e^{l_t}
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          Frag<IO> fa;
          fa.load8(s.sC + (16 * rb + c) * LDN + 32 * ns + 8 * g);
#pragma unroll
          for (int pb = 0; pb < PB; ++pb) {
            Frag<IO> fb;
            fb.load8(s.sH + (16 * pb + c) * LDN + 32 * ns + 8 * g);
            mma(Y[pb], fa, fb);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tq = (16 * rb + 4 * g + i) >> lgR;
          const float sc = exp2f(s.sTok[tq < Q ? tq : Q - 1].y);
#pragma unroll
          for (int pb = 0; pb < PB; ++pb) Y[pb][i] *= sc;
        }
        // intra-chunk term: (S . M) X over 32-key slabs up to the diagonal
        const int tq_c = (16 * rb + c) >> lgR;          // query token of this lane's S^T column
        const float lq_c = s.sTok[tq_c < Q ? tq_c : Q - 1].y;
        const int nks = (16 * rb + 15) / 32 + 1;
        for (int ks = 0; ks < nks; ++ks) {
          Frag<IO> fsm;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int kb = 2 * ks + half;
            f32x4 St = f32x4{0.f, 0.f, 0.f, 0.f};
            if (kb <= rb) {
#pragma unroll
              for (int ns = 0; ns < NS; ++ns) {
                Frag<IO> fa, fb;
                fa.load8(s.sB + (16 * kb + c) * LDN + 32 * ns + 8 * g);
                fb.load8(s.sC + (16 * rb + c) * LDN + 32 * ns + 8 * g);
                mma(St, fa, fb);
              }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tk = (16 * kb + 4 * g + i) >> lgR;
              float m = 0.f;
              if (kb <= rb && tk <= tq_c) {
                const float4 kt = s.sTok[tk];
                m = kt.x * exp2f(lq_c - kt.y);
                if (tk < tq_c) m += kt.z * exp2f(lq_c - kt.w);
              }
              fsm.set(4 * half + i, St[i] * m);
            }
          }
#pragma unroll
          for (int pb = 0; pb < PB; ++pb) {
            Frag<IO> fx;
            const IO* xr = s.sXt + (16 * pb + c) * ldr + 32 * ks + 4 * g;
            fx.load44(xr, xr + 16);
            mma(Y[pb], fsm, fx);
          }
        }
        // skip term D x, then store the valid rows
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
          float xv[4];
          load4(s.sXt + (16 * pb + c) * ldr + 16 * rb + 4 * g, xv);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rho = 16 * rb + 4 * g + i;
            const int t = rho >> lgR, r = rho & (R - 1);
            if (t < Lc) Yg[(size_t)(c0 + t) * tokX + r * P + 16 * pb + c] = from_f32<IO>(Y[pb][i] + Dh * xv[i]);
          }
        }
      }
      __syncthreads();  // all reads of sH done before it is overwritten below
    }

    // ---------------- C: state update and rotation to the next frame ----------------
    {
      const float decE = expf(s.sMisc[0]);
      const int nks = rows_pad / 32;
      const bool last_chunk = (ck == ck1 - 1);
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int tile = wave + k * kWaves;
        if (tile < NT) {
          const int nb = tile / PB, pb = tile % PB;
          f32x4 acc = Hreg[k] * decE;
          for (int ks = 0; ks < nks; ++ks) {
            Frag<IO> fa, fb;
            fa.load8(s.sBt + (16 * nb + c) * ldr + 32 * ks + 8 * g);
            fb.load8(s.sXt + (16 * pb + c) * ldr + 32 * ks + 8 * g);
            mma(acc, fa, fb);
          }
          // rows n = 16nb + 4g + i: pairs (8nb + 2g) and (8nb + 2g + 1) -> lane-local rotation
          const float2 r0 = s.sEnd[8 * nb + 2 * g];
          const float2 r1 = s.sEnd[8 * nb + 2 * g + 1];
          float v[4] = {acc[0], acc[1], acc[2], acc[3]};
          rot2(v[0], v[1], r0.x, r0.y);
          rot2(v[2], v[3], r1.x, r1.y);
          Hreg[k] = f32x4{v[0], v[1], v[2], v[3]};
          const int p = 16 * pb + c, n0 = 16 * nb + 4 * g;
          store4(s.sH + p * LDN + n0, v);
          if (last_chunk) {
            if (writes_final) {
              store4(a.h + ((size_t)chain * P + p) * N + n0, v);
            } else if (mode == kSummary) {
              store4(a.seg_state + (((size_t)seg * kp.batch * H + chain) * P + p) * N + n0, v);
            }
          }
        }
      }
      if (mode == kSummary) {
        // running angle total of the segment (pairs); sPhi[te] is this chunk's total
        for (int j = tid; j < N / 2; j += kThreads) {
          const float tot = reduce_angle(s.sSeg[j] + s.sPhi[te * (N / 2) + j]);
          s.sSeg[j] = tot;
          if (last_chunk) a.seg_angle[((size_t)seg * kp.batch * H + chain) * (N / 2) + j] = tot;
        }
        if (tid == 0 && last_chunk) a.seg_decay[(size_t)seg * kp.batch * H + chain] = lsum;
      }
    }
  }

  // pending pair of the last token
  if (writes_final) {
    const IO* Bl = Bg + (size_t)(T - 1) * tokBC;
    const IO* Xl = Xg + (size_t)(T - 1) * tokX;
    IO* Bp = static_cast<IO*>(a.B_prev) + (size_t)chain * R * N;
    IO* Xp = static_cast<IO*>(a.x_prev) + (size_t)chain * R * P;
    __syncthreads();  // every thread's read of the old pending (entry value) is long done
    for (int e = tid; e < R * N; e += kThreads) Bp[e] = Bl[e];
    for (int e = tid; e < R * P; e += kThreads) Xp[e] = Xl[e];
  }
}

// ----------------------------------------------------------------------------
// Segment scan: entry values E_g of every segment from the summaries.
//   E_0     = alpha_0 h_0 + beta_0 x_prev (x) B_prev            (from the state)
//   E_{g+1} = e^{L_g} Rot(Phi_g) E_g + W_g                      (affine map per pair)
// One lane per segment: an inclusive wave-level scan composes the maps
// (rho, w) with (rho_b, w_b) o (rho_a, w_a) = (rho_b rho_a, rho_b w_a + w_b),
// rho = e^{L + i Phi} kept in polar form.  Each wave handles 64/G2 (p, pair)
// elements of one chain, G2 = nseg rounded up to a power of two.
// ----------------------------------------------------------------------------
template <typename IO>
__global__ __launch_bounds__(256) void segment_scan_kernel(PrefillArgs a, int batch, int H, int P, int N, int R,
                                                           int G2) {
  const int nseg = a.nseg;
  const int chains = batch * H;
  const int lane = threadIdx.x & 63;
  const int per_wave = 64 / G2;
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;  // global wave index
  const int sub = lane / G2;                                     // element within the wave
  const int gseg = lane % G2;                                    // segment of this lane
  const long long elem = (long long)gw * per_wave + sub;         // over chains * P * N/2
  const long long nelem = (long long)chains * P * (N / 2);
  const bool active = elem < nelem;
  const long long el = active ? elem : nelem - 1;  // past the end: the last element's chain
  const int chain = (int)(el / ((long long)P * (N / 2)));
  const int rem = (int)(el % ((long long)P * (N / 2)));
  const int p = rem / (N / 2), j = rem % (N / 2);
  const int hh = chain % H;
  const size_t seg_stride = (size_t)chains;

  // BC normalisation of the pending B_prev rows: a wave's elements all belong
  // to one chain (P * N/2 is a multiple of the elements per wave), so the
  // wave sums each row's squares together (lane l: columns l, l + 64).
  float bscale[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
  if (a.nbw) {
    const IO* Bp = static_cast<const IO*>(a.B_prev) + (size_t)chain * R * N;
#pragma unroll
    for (int r = 0; r < 8; ++r) {  // R <= 8
      if (r < R) {
        float ss = 0.f;
        for (int n = lane; n < N; n += 64) {
          const float v = to_f32(Bp[r * N + n]);
          ss += v * v;
        }
        ss = lane_group_sum(ss, 64);
        bscale[r] = rsqrtf(ss / (float)N + a.neps);
      }
    }
  }
  // E_0 from the state (only the lane of segment 0 needs it).
  float e0r = 0.f, e0i = 0.f;
  if (active && gseg == 0) {
    const int b = chain / H;
    const float dt0 = a.dt[(size_t)b * a.seqlen * H + hh];
    const float lm0 = a.lam[(size_t)b * a.seqlen * H + hh];
    const float alpha0 = expf(dt0 * a.A[hh]);
    const float beta0 = input_weights(dt0, lm0, alpha0, a.disc).x;
    const float* hp = a.h + ((size_t)chain * P + p) * N + 2 * j;
    e0r = alpha0 * hp[0];
    e0i = alpha0 * hp[1];
    const IO* Bp = static_cast<const IO*>(a.B_prev) + (size_t)chain * R * N;
    const IO* Xp = static_cast<const IO*>(a.x_prev) + (size_t)chain * R * P;
    const float g0 = a.nbw ? a.nbw[(size_t)hh * N + 2 * j] : 1.f;
    const float g1 = a.nbw ? a.nbw[(size_t)hh * N + 2 * j + 1] : 1.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {  // R <= 8
      if (r < R) {
        const float xp = beta0 * to_f32(Xp[r * P + p]) * bscale[r];
        e0r += xp * g0 * to_f32(Bp[r * N + 2 * j]);
        e0i += xp * g1 * to_f32(Bp[r * N + 2 * j + 1]);
      }
    }
  }
  // Map of segment g (g < nseg-1): (L_g, Phi_g, W_g); identity elsewhere.
  float Lg = 0.f, Pg = 0.f, wr = 0.f, wi = 0.f;
  if (active && gseg < nseg - 1) {
    const size_t cs = (size_t)gseg * seg_stride + chain;
    Lg = a.seg_decay[cs];
    Pg = a.seg_angle[cs * (N / 2) + j];
    const float* wp = a.seg_state + (cs * P + p) * N + 2 * j;
    wr = wp[0];
    wi = wp[1];
  }
  // inclusive scan over the G2 lanes of this element
  for (int d = 1; d < G2; d <<= 1) {
    const float uL = __shfl_up(Lg, d, G2);
    const float uP = __shfl_up(Pg, d, G2);
    const float ur = __shfl_up(wr, d, G2);
    const float ui = __shfl_up(wi, d, G2);
    if (gseg >= d) {
      // this lane's map (b) composed after the earlier map (a = u)
      float sn, cs;
      sincosf(Pg, &sn, &cs);
      const float mag = expf(Lg);
      const float nr = mag * (cs * ur - sn * ui) + wr;
      const float ni = mag * (sn * ur + cs * ui) + wi;
      wr = nr;
      wi = ni;
      Lg += uL;
      Pg += uP;
    }
  }
  // E_{g+1} = composed_{0..g}(E_0), written to slot g+1; slot 0 gets E_0.
  const float e0r_b = __shfl(e0r, 0, G2);
  const float e0i_b = __shfl(e0i, 0, G2);
  if (!active) return;
  float sn, cs;
  sincosf(Pg, &sn, &cs);
  const float mag = expf(Lg);
  const float er = mag * (cs * e0r_b - sn * e0i_b) + wr;
  const float ei = mag * (sn * e0r_b + cs * e0i_b) + wi;
  if (gseg == 0) {
    float* d0 = a.seg_state + ((size_t)chain * P + p) * N + 2 * j;
    // slot 0 (W_0 already consumed by every lane above)
    d0[0] = e0r_b;
    d0[1] = e0i_b;
  }
  if (gseg + 1 < nseg) {
    float* d = a.seg_state + (((size_t)(gseg + 1) * seg_stride + chain) * P + p) * N + 2 * j;
    d[0] = er;
    d[1] = ei;
  }
}

template <typename IO, int N, int P>
hipError_t launch_fused_t(const Dims& d, const PrefillArgs& a, hipStream_t st) {
  const int rows = d.Q * d.R;
  const int rows_pad = (rows + 31) & ~31;
  const size_t lds = Lds<IO, N, P>::bytes(rows_pad, d.Q);
  static bool attr_set = false;
  if constexpr (Limits<IO, N, P>::kMaxRows > 0) {
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<IO, N, P>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  KParams kp;
  kp.a = a;
  kp.batch = d.batch;
  kp.heads = d.heads;
  kp.R = d.R;
  kp.lgR = d.R == 1 ? 0 : (d.R == 2 ? 1 : 2);
  kp.Q = d.Q;
  const int chains = d.batch * d.heads;
  const bool pc = prefill_pc_supported(d);
  // the epilogue and the BC normalisation live in the producer/consumer
  // kernel, and so do padded ranks (the host checks all this first)
  if ((a.gz || a.nbw) && !pc) return hipErrorInvalidValue;
  if (!pc && !(d.R == 1 || d.R == 2 || d.R == 4)) return hipErrorInvalidValue;
  auto pass = [&](int mode, int nblocks) -> hipError_t {
    if (pc) return launch_prefill_pc(d, a, st, mode, nblocks);
    if constexpr (Limits<IO, N, P>::kMaxRows == 0) {
      return hipErrorInvalidValue;  // (never: such tiles fit at no height, which the host checks first)
    } else {
      kp.mode = mode;
      kp.nblocks = nblocks;
      hipLaunchKernelGGL((prefill_kernel<IO, N, P>), dim3(nblocks), dim3(kThreads), lds, st, kp);
      return hipGetLastError();
    }
  };
  if (a.nseg <= 1) return pass(kFused, chains);
  // pass 1: summaries of segments 0 .. nseg-2 from a zero entry value
  hipError_t e = pass(kSummary, chains * (a.nseg - 1));
  if (e != hipSuccess) return e;
  // pass 2: scan over segments -> entry values
  int G2 = 1;
  while (G2 < a.nseg) G2 <<= 1;
  const long long nelem = (long long)chains * d.P * (d.N / 2);
  const long long waves = (nelem + (64 / G2) - 1) / (64 / G2);
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  hipLaunchKernelGGL((segment_scan_kernel<IO>), dim3(blocks), dim3(256), 0, st, a, d.batch, d.heads, d.P, d.N,
                     d.R, G2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // pass 3: every segment from its entry value
  return pass(kSegment, chains * a.nseg);
}

template <typename IO, int N>
hipError_t launch_p(const Dims& d, const PrefillArgs& a, hipStream_t s) {
  switch (d.P) {
    case 16: return launch_fused_t<IO, N, 16>(d, a, s);
    case 32: return launch_fused_t<IO, N, 32>(d, a, s);
    case 64: return launch_fused_t<IO, N, 64>(d, a, s);
    default: return launch_fused_t<IO, N, 128>(d, a, s);
  }
}

template <typename IO>
hipError_t launch_n(const Dims& d, const PrefillArgs& a, hipStream_t s) {
  switch (d.N) {
    case 16: return launch_p<IO, 16>(d, a, s);
    case 32: return launch_p<IO, 32>(d, a, s);
    case 64: return launch_p<IO, 64>(d, a, s);
    case 128: return launch_p<IO, 128>(d, a, s);
    default: return launch_p<IO, 256>(d, a, s);
  }
}

template <typename IO>
int max_rows(const Dims& d) {
  switch (d.N * 1000 + d.P) {
#define M3_CASE(NN, PP) \
  case NN * 1000 + PP: return Limits<IO, NN, PP>::kMaxRows;
    M3_CASE(16, 16) M3_CASE(16, 32) M3_CASE(16, 64) M3_CASE(16, 128)
    M3_CASE(32, 16) M3_CASE(32, 32) M3_CASE(32, 64) M3_CASE(32, 128)
    M3_CASE(64, 16) M3_CASE(64, 32) M3_CASE(64, 64) M3_CASE(64, 128)
    M3_CASE(128, 16) M3_CASE(128, 32) M3_CASE(128, 64) M3_CASE(128, 128)
    M3_CASE(256, 16) M3_CASE(256, 32) M3_CASE(256, 64) M3_CASE(256, 128)
#undef M3_CASE
    default: return 0;
  }
}

}  // namespace

namespace {
// Whether the single-role kernel's tiles fit at d.Q (it takes ranks 1, 2
// and 4 only: its rows are (token, rank) pairs with no padded ranks).
bool single_role_fits(const Dims& d) {
  if (!(d.R == 1 || d.R == 2 || d.R == 4)) return false;
  if ((d.Q / 4) * (d.N / 8) > kThreads) return false;  // one angle item (4 tokens x 4 pairs) per thread
  const int rows_pad = ((d.Q * d.R) + 31) & ~31;
  return rows_pad <= (d.bf16 ? max_rows<bf16>(d) : max_rows<float>(d));
}
}  // namespace

int prefill_tile_chunk(const Dims& d) {
  // The chunk length is a tile height: the chunked form gives the same result
  // for any chunk length.  The producer/consumer kernel at the largest height
  // <= Q whose tiles fit (halving down to 16 tokens, or to 4 when a token
  // brings 4 or 8 tile rows), else the single-role kernel likewise (down to
  // 16); 0 when neither fits at any height.  Support is thereby monotone in
  // the chunk: whatever runs at chunk 16 runs at 32 and 64.
  const int qmin = d.R > 2 ? 4 : 16;
  for (int q = d.Q; q >= qmin; q /= 2) {
    Dims e = d;
    e.Q = q;
    if (prefill_pc_supported(e)) return q;
  }
  for (int q = d.Q; q >= 16; q /= 2) {
    Dims e = d;
    e.Q = q;
    if (single_role_fits(e)) return q;
  }
  return 0;
}

bool prefill_supported(const Dims& d) {
  const bool n_ok = d.N == 16 || d.N == 32 || d.N == 64 || d.N == 128 || d.N == 256;
  const bool p_ok = d.P == 16 || d.P == 32 || d.P == 64 || d.P == 128;
  const bool r_ok = d.R >= 1 && d.R <= 8;
  const bool q_ok = d.Q == 16 || d.Q == 32 || d.Q == 64;
  if (!(n_ok && p_ok && r_ok && q_ok)) return false;
  return prefill_tile_chunk(d) > 0;
}

bool prefill_pc_path_supported(const Dims& d) {
  Dims e = d;
  e.Q = prefill_tile_chunk(d);
  return e.Q > 0 && prefill_pc_supported(e);
}

hipError_t launch_prefill(const Dims& d, const PrefillArgs& a, hipStream_t s) {
  return d.bf16 ? launch_n<bf16>(d, a, s) : launch_n<float>(d, a, s);
}

}  // namespace m3
