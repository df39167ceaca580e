// Mamba-3 chunked prefill for gfx950: producer/consumer form.
//
// Same algebra as the single-role kernel in m3_prefill.hip (chunked "dual"
// form of the exponential-trapezoid recurrence with rotating state; lilting.ch
// Mamba-3 article, "アーキテクチャ改善" 1-3, and its SSM-history section on the
// matmul-shaped restructuring): per chunk, with local angles phi and local
// log-decay l,
//     y^T[p][t]  = e^{l_t} (E^T Ct^T)[p][t] + (X^T (S.M)^T)[p][t]    (+ D x on the diagonal of S.M)
//     E'         = Rot(phi_e) [ e^{l_E} E + Bt^T diag(w) X ]
// where E is the chunk's entry value (the carried lab-frame state with the
// first token's decay and previous-input term applied), S^T = Bt Ct^T, and M
// the trapezoid decay mask.
//
// One workgroup of 8 waves per chain (or chain segment):
//   waves 0-3 produce: stream dt, lam, theta, B, C, x for chunk i+1 / i+2 from
//     HBM into registers (16-byte loads, addresses clamped so every load is
//     unconditional), run the in-chunk decay scan and angle prefix, rotate B
//     and C, and write chunk i's bf16/fp32 tiles into LDS buffer i%2;
//   waves 4-7 consume chunk i-1 from buffer (i-1)%2 on the matrix cores.  Each
//     consumer wave owns 16-column slices (p-blocks) of the P x N state, kept
//     in fp32 registers as E^T tiles (rows n, columns p).  Because the K order
//     inside an MFMA is free as long as both operands agree, the state tiles
//     feed the carried-state product E^T Ct^T directly (two adjacent n-tiles
//     give one 32-wide K slab), and the masked score tile S^T leaves its
//     accumulator as the B operand of X^T (S.M)^T; the output comes out as
//     y^T, so each lane stores 4 consecutive p of one token (8-byte stores).
// A single workgroup barrier per chunk separates the roles' buffers: tiles
// are double buffered, per-token coefficients triple buffered (written one
// chunk ahead by the producers, read by producers in the next chunk and by
// consumers in the one after).
#include "m3_kernels.hpp"
#include "m3_mfma.hpp"

namespace m3 {
namespace {

constexpr int kPcThreads = 512;
constexpr int kProdThreads = 256;
constexpr int kConsWaves = 4;
constexpr float kLog2ePc = 1.4426950408889634f;

enum PcMode : int { kPcFused = 0, kPcSummary = 1, kPcSegment = 2 };

struct PcParams {
  PrefillArgs a;
  int batch, heads, R, lgR, Q;
  int mode;
  int nblocks;
};

__device__ __forceinline__ int pc_remap_block(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

// LDS layout for <IO, N, P> at runtime rows_pad (= Q*R rounded up to 32).
template <typename IO, int N, int P>
struct PcLds {
  static constexpr int E = sizeof(IO);
  static constexpr int PAD = 16 / E;
  static constexpr int NK = N < 32 ? 32 : N;
  static constexpr int LDN = NK + PAD;
  // one tile buffer
  __host__ __device__ static constexpr size_t buf_bytes(int rows_pad) {
    return (size_t)rows_pad * LDN * E * 2            // sB, sC
           + (size_t)N * (rows_pad + PAD) * E        // sBt
           + (size_t)P * (rows_pad + PAD) * E        // sXt
           + (size_t)(N / 2) * 16;                   // sEnd {cos, sin, phi, 0}
  }
  __host__ __device__ static constexpr size_t coef_bytes(int Q) { return (size_t)Q * 20 + 16; }
  __host__ __device__ static constexpr size_t bytes(int rows_pad, int Q) {
    return 2 * buf_bytes(rows_pad) + 3 * coef_bytes(Q) + (N / 2) * 4;
  }
};

template <typename IO, int N, int P>
struct PcBuf {
  IO *sB, *sC, *sBt, *sXt;
  float4* sEnd;
};
struct PcCoef {
  float4* sTok;  // [Q] {gamma, l*log2e, beta of the next token, l_next*log2e}
  float* sW;     // [Q] state-update weights
  float* sMisc;  // [0] l_E, [1] l_E*log2e
};

// Largest padded row count and register-array bounds of an instance.
template <typename IO, int N, int P>
struct PcLimits {
  static constexpr int NK = PcLds<IO, N, P>::NK;
  static constexpr bool fits(int r) {
    return PcLds<IO, N, P>::bytes(r, r < 64 ? r : 64) <= 160 * 1024 && r * NK * (int)sizeof(IO) <= 16384 &&
           (r / 4) * (N / 8) <= 2 * kProdThreads && (r / 4) * (P / 8) <= 2 * kProdThreads;
  }
  static constexpr int kMaxRows = fits(128) ? 128 : fits(64) ? 64 : fits(32) ? 32 : 0;
  static constexpr int kMaxRB = kMaxRows / 16;                                    // row blocks
  static constexpr int kMI = (kMaxRows / 4) * (N / 8) > kProdThreads ? 2 : 1;     // B/C items per thread
  static constexpr int kMX = (kMaxRows / 4) * (P / 8) > kProdThreads ? 2 : 1;     // x items per thread
  static constexpr int kPBW = (P / 16 + kConsWaves - 1) / kConsWaves;            // p-blocks per consumer
};

template <typename IO, int N, int P>
__global__ __launch_bounds__(kPcThreads, 1) void prefill_pc_kernel(PcParams kp) {
  using L = PcLds<IO, N, P>;
  using Lim = PcLimits<IO, N, P>;
  constexpr int NB = N / 16, PB = P / 16;
  constexpr int NK = L::NK, LDN = L::LDN, PAD = L::PAD;
  constexpr int NS = NK / 32;
  constexpr int MI = Lim::kMI, MX = Lim::kMX, PBW = Lim::kPBW, RBM = Lim::kMaxRB;
  extern __shared__ __align__(16) char smem[];

  const PrefillArgs& a = kp.a;
  const int Q = kp.Q, R = kp.R, lgR = kp.lgR, H = kp.heads;
  const int T = a.seqlen;
  const int mode = kp.mode;
  const int nseg_grid = (mode == kPcFused) ? 1 : (mode == kPcSummary ? a.nseg - 1 : a.nseg);
  const int bid = pc_remap_block(blockIdx.x, kp.nblocks);
  const int chain = bid / nseg_grid;
  const int seg = bid % nseg_grid;
  const int b = chain / H, hh = chain % H;
  const int nchunks = (T + Q - 1) / Q;
  const int ck0 = (mode == kPcFused) ? 0 : seg * a.seg_chunks;
  int ck1 = (mode == kPcFused) ? nchunks : ck0 + a.seg_chunks;
  if (ck1 > nchunks) ck1 = nchunks;
  const bool writes_final = (mode == kPcFused) || (mode == kPcSegment && seg == a.nseg - 1);
  const bool has_y = mode != kPcSummary;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const bool producer = wave < 4;
  const int rows = Q * R;
  const int rows_pad = (rows + 31) & ~31;
  const int ldr = rows_pad + PAD;

  // ---- LDS: [tile buffer 0 | tile buffer 1 | coefs x3 | sSeg] ----
  const size_t bufB = (size_t)rows_pad * LDN * sizeof(IO);           // sB, sC
  const size_t bufBt = (size_t)N * ldr * sizeof(IO);
  const size_t bufXt = (size_t)P * ldr * sizeof(IO);
  const size_t bufStride = 2 * bufB + bufBt + bufXt + (size_t)(N / 2) * 16;
  const size_t coefStride = (size_t)Q * 20 + 16;
  char* const coefBase = smem + 2 * bufStride;
  float* const sSeg = reinterpret_cast<float*>(coefBase + 3 * coefStride);
  auto getbuf = [&](int ck) {
    char* p = smem + (size_t)(ck & 1) * bufStride;
    PcBuf<IO, N, P> r;
    r.sB = reinterpret_cast<IO*>(p);
    r.sC = reinterpret_cast<IO*>(p + bufB);
    r.sBt = reinterpret_cast<IO*>(p + 2 * bufB);
    r.sXt = reinterpret_cast<IO*>(p + 2 * bufB + bufBt);
    r.sEnd = reinterpret_cast<float4*>(p + 2 * bufB + bufBt + bufXt);
    return r;
  };
  auto getcoef = [&](int ck) {
    char* p = coefBase + (size_t)(ck % 3) * coefStride;
    PcCoef r;
    r.sTok = reinterpret_cast<float4*>(p);
    r.sW = reinterpret_cast<float*>(p + (size_t)Q * 16);
    r.sMisc = reinterpret_cast<float*>(p + (size_t)Q * 20);
    return r;
  };
  if (NK != N) {
    // columns N .. NK-1 of sB and sC are never written: keep them zero
    for (int k = 0; k < 2; ++k) {
      const PcBuf<IO, N, P> bk = getbuf(k);
      for (int e = tid; e < rows_pad * LDN; e += kPcThreads) {
        bk.sB[e] = from_f32<IO>(0.f);
        bk.sC[e] = from_f32<IO>(0.f);
      }
    }
  }
  if (mode == kPcSummary)
    for (int j = tid; j < N / 2; j += kPcThreads) sSeg[j] = 0.f;

  const float Ah = a.A[hh];
  const float Dh = a.D[hh];
  const size_t tokBC = (size_t)H * R * N;
  const size_t tokX = (size_t)H * R * P;
  const size_t tokTh = (size_t)H * (N / 2);
  const IO* Bg = static_cast<const IO*>(a.B) + ((size_t)b * T * H + hh) * R * N;
  const IO* Cg = static_cast<const IO*>(a.C) + ((size_t)b * T * H + hh) * R * N;
  const IO* Xg = static_cast<const IO*>(a.x) + ((size_t)b * T * H + hh) * R * P;
  IO* Yg = static_cast<IO*>(a.y) + ((size_t)b * T * H + hh) * R * P;
  const float* THg = a.theta + ((size_t)b * T * H + hh) * (N / 2);
  const float* DTg = a.dt + (size_t)b * T * H + hh;
  const float* LMg = a.lam + (size_t)b * T * H + hh;

  auto chunk_len = [&](int ck) { return (T - ck * Q < Q) ? (T - ck * Q) : Q; };

  if (producer) {
    // ======================= producers (waves 0-3) =======================
    // Item = (row group rg: 4 consecutive (token, rank) rows, pair group pg:
    // 4 state pairs = 8 columns).  Items are laid out row-group-fastest, so the
    // RG = rows_pad/4 row groups of one pair group are RG consecutive lanes of
    // one wave and the angle prefix over the chunk is an in-wave segmented scan.
    const int pt = tid;
    const int RG = rows_pad / 4;
    const int npg = N / 8;
    const int nbitems = RG * npg;
    const int npx = P / 8;
    const int nxitems = RG * npx;
    const int ntok = 4 >> lgR;  // tokens per row group (R <= 4)
    Raw8<IO> rb_[MI][4], rc_[MI][4], rx_[MX][4];  // raw B, C, x of the next chunk
    float4 rth[MI][4];                            // raw theta of the next chunk
    float rdt = 0.f, rlm = 0.f, rdtn = 0.f, rlmn = 0.f;  // raw dt/lam (wave 0), chunk after next

    auto load_chunk = [&](int ck) {  // B, C, x, theta of chunk ck
      const int c0 = ck * Q, Lc = chunk_len(ck);
#pragma unroll
      for (int m = 0; m < MI; ++m) {
        const int it = pt + m * kProdThreads;
        if (it < nbitems) {
          const int rg = it % RG, pg = it / RG;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rho = 4 * rg + k;
            const bool valid = rho < rows && (rho >> lgR) < Lc;
            const int t = valid ? (rho >> lgR) : 0, r = valid ? (rho & (R - 1)) : 0;
            rb_[m][k].load(Bg + (size_t)(c0 + t) * tokBC + r * N + 8 * pg);
            if (has_y) rc_[m][k].load(Cg + (size_t)(c0 + t) * tokBC + r * N + 8 * pg);
          }
          const int t0 = (4 * rg) >> lgR;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int t = t0 + (q < ntok ? q : ntok - 1);
            t = t < Lc ? t : 0;
            rth[m][q] = *reinterpret_cast<const float4*>(THg + (size_t)(c0 + t) * tokTh + 4 * pg);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MX; ++m) {
        const int it = pt + m * kProdThreads;
        if (it < nxitems) {
          const int rg = it % RG, xg = it / RG;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rho = 4 * rg + k;
            const bool valid = rho < rows && (rho >> lgR) < Lc;
            const int t = valid ? (rho >> lgR) : 0, r = valid ? (rho & (R - 1)) : 0;
            rx_[m][k].load(Xg + (size_t)(c0 + t) * tokX + r * P + 8 * xg);
          }
        }
      }
    };
    auto load_dt = [&](int ck) {  // dt, lam of chunk ck and of the token after it (wave 0)
      if (wave != 0) return;
      const int c0 = ck * Q, Lc = chunk_len(ck);
      const int t = lane < Lc ? lane : Lc - 1;
      rdt = DTg[(size_t)(c0 + t) * H];
      rlm = LMg[(size_t)(c0 + t) * H];
      const int tn = (c0 + Lc < T) ? c0 + Lc : c0 + Lc - 1;
      rdtn = DTg[(size_t)tn * H];
      rlmn = LMg[(size_t)tn * H];
    };
    // In-chunk decay scan and per-token coefficients of chunk ck -> coef slot ck % 3.
    // sTok[t] = {A_t, B_t, L_t, 0} with L_t = l_t log2(e) and the mask weights
    // gamma_t 2^{L_q - L_t} = 2^{L_q - A_t},  beta_{t+1} 2^{L_q - L_{t+1}} = 2^{L_q - B_t}
    // (a zero weight gives an infinite exponent and an exact zero).
    auto decay_coefs = [&](int ck) {
      if (wave != 0) return;
      const int c0 = ck * Q, Lc = chunk_len(ck);
      const bool fold_next = c0 + Lc < T;
      const PcCoef co = getcoef(ck);
      const int t = lane;
      const bool valid = t < Lc;
      const float dtv = valid ? rdt : 0.f, lmv = valid ? rlm : 0.f;
      const float av = (valid && t > 0) ? dtv * Ah : 0.f;
      const float ell = wave_inclusive_scan(av);
      const float gam = lmv * dtv;
      const float bet = (1.0f - lmv) * dtv;
      const float dtn = fold_next ? rdtn : 0.f, lmn = fold_next ? rlmn : 0.f;
      const float ell_last = __shfl(ell, Lc - 1, kWave);
      const float ellE = ell_last + dtn * Ah;
      const float bet_up = __shfl_down(bet, 1, kWave);
      const float ell_up = __shfl_down(ell, 1, kWave);
      float betn, elln;
      if (t < Lc - 1) {
        betn = bet_up;
        elln = ell_up;
      } else if (t == Lc - 1) {
        betn = (1.0f - lmn) * dtn;
        elln = ellE;
      } else {
        betn = 0.f;
        elln = ellE;
      }
      const float ellv = valid ? ell : ell_last;
      const float w = valid ? (gam * expf(ellE - ellv) + betn * expf(ellE - elln)) : 0.f;
      const float inf = __builtin_huge_valf();
      const float L2 = ellv * kLog2ePc;
      const float Ak = (valid && gam > 0.f) ? L2 - __log2f(gam) : inf;
      const float Bk = (valid && betn > 0.f) ? elln * kLog2ePc - __log2f(betn) : inf;
      if (t < Q) {
        co.sTok[t] = make_float4(Ak, Bk, L2, 0.f);
        co.sW[t] = w;
      }
      if (t == 0) {
        co.sMisc[0] = ellE;
        co.sMisc[1] = ellE * kLog2ePc;
      }
    };
    // Angles (in-wave scan), rotation, and the tiles of chunk ck -> tile buffer ck % 2.
    auto build_tiles = [&](int ck) {
      const int Lc = chunk_len(ck);
      const int te = Lc - 1;
      const PcBuf<IO, N, P> bf = getbuf(ck);
      const float* sW = getcoef(ck).sW;
#pragma unroll
      for (int m = 0; m < MI; ++m) {
        const int it = pt + m * kProdThreads;
        if (it < nbitems) {
          const int rg = it % RG, pg = it / RG;
          const int t0 = (4 * rg) >> lgR;
          float th[4][4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool tv = q < ntok && t0 + q < Lc;
            th[q][0] = tv ? rth[m][q].x : 0.f;
            th[q][1] = tv ? rth[m][q].y : 0.f;
            th[q][2] = tv ? rth[m][q].z : 0.f;
            th[q][3] = tv ? rth[m][q].w : 0.f;
          }
          // exclusive prefix of the row groups' totals within the pair group
          float base[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float tot = th[0][j] + th[1][j] + th[2][j] + th[3][j];
            float inc = tot;
            for (int d = 1; d < RG; d <<= 1) {
              const float u = __shfl_up(inc, d, RG);
              if (rg >= d) inc += u;
            }
            base[j] = inc - tot;
          }
          float bt[4][8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rho = 4 * rg + k;
            const int t = rho >> lgR;
            const int kq = t - t0;  // token of this row within the row group
            const bool valid = rho < rows && t < Lc;
            float ph[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float acc = base[j];
#pragma unroll
              for (int q = 0; q < 4; ++q) acc += (q <= kq) ? th[q][j] : 0.f;
              ph[j] = acc;
            }
            float bv[8], cv[8];
            rb_[m][k].unpack(bv);
            if (has_y) rc_[m][k].unpack(cv);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float sn, cs;
              trig<IO>(ph[j], sn, cs);
              rot2(bv[2 * j], bv[2 * j + 1], cs, -sn);
              if (has_y) rot2(cv[2 * j], cv[2 * j + 1], cs, -sn);
            }
            const float wt = valid ? sW[t] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              bv[e] = valid ? bv[e] : 0.f;
              cv[e] = (valid && has_y) ? cv[e] : 0.f;
              bt[k][e] = bv[e] * wt;
            }
            store8(bf.sB + rho * LDN + 8 * pg, bv);
            if (has_y) store8(bf.sC + rho * LDN + 8 * pg, cv);
            if (valid && t == te && (rho & (R - 1)) == 0) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                float sn, cs;
                sincosf(ph[j], &sn, &cs);
                bf.sEnd[4 * pg + j] = make_float4(cs, sn, ph[j], 0.f);
              }
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float col[4] = {bt[0][e], bt[1][e], bt[2][e], bt[3][e]};
            store4(bf.sBt + (8 * pg + e) * ldr + 4 * rg, col);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MX; ++m) {
        const int it = pt + m * kProdThreads;
        if (it < nxitems) {
          const int rg = it % RG, xg = it / RG;
          float xv[4][8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rho = 4 * rg + k;
            const bool valid = rho < rows && (rho >> lgR) < Lc;
            rx_[m][k].unpack(xv[k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[k][e] = valid ? xv[k][e] : 0.f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float col[4] = {xv[0][e], xv[1][e], xv[2][e], xv[3][e]};
            store4(bf.sXt + (8 * xg + e) * ldr + 4 * rg, col);
          }
        }
      }
    };

    if (ck0 < ck1) {
      // prologue: coefficients of the first chunk, then the first prefetches
      load_dt(ck0);
      decay_coefs(ck0);
      load_chunk(ck0);
      if (ck0 + 1 < ck1) load_dt(ck0 + 1);
    }
    __syncthreads();
    for (int i = ck0; i <= ck1; ++i) {
      if (i < ck1) {
        build_tiles(i);
        if (i + 1 < ck1) {
          decay_coefs(i + 1);
          load_chunk(i + 1);
          if (i + 2 < ck1) load_dt(i + 2);
        }
      }
      __syncthreads();
    }
  } else {
    // ======================= consumers (waves 4-7) =======================
    const int cw = wave - 4;
    f32x4 Hreg[PBW][NB];  // E^T tiles: rows n = 16nb + 4g + i, column p = 16pb + c
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < PBW; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) Hreg[u][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      float alpha0 = 0.f, beta0 = 0.f;
      if (mode == kPcFused) {
        const float dt0 = DTg[0];
        const float lm0 = LMg[0];
        alpha0 = expf(dt0 * Ah);
        beta0 = (1.0f - lm0) * dt0;
      }
#pragma unroll
      for (int u = 0; u < PBW; ++u) {
        const int pb = cw + kConsWaves * u;
        if (pb < PB) {
          const int p = 16 * pb + c;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int n0 = 16 * nb + 4 * g;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (mode == kPcFused) {
              float h0[4];
              load4(a.h + ((size_t)chain * P + p) * N + n0, h0);
              const IO* Bp = static_cast<const IO*>(a.B_prev) + (size_t)chain * R * N;
              const IO* Xp = static_cast<const IO*>(a.x_prev) + (size_t)chain * R * P;
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) v[i4] = alpha0 * h0[i4];
              for (int r = 0; r < R; ++r) {
                float bp[4];
                load4(Bp + r * N + n0, bp);
                const float xp = beta0 * to_f32(Xp[r * P + p]);
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) v[i4] += xp * bp[i4];
              }
            } else if (mode == kPcSegment) {
              load4(a.seg_state + (((size_t)seg * kp.batch * H + chain) * P + p) * N + n0, v);
            }
            Hreg[u][nb] = f32x4{v[0], v[1], v[2], v[3]};
          }
        }
      }
    }
    __syncthreads();
    for (int i = ck0; i <= ck1; ++i) {
      if (i > ck0) {
        const int j = i - 1;
        const int c0 = j * Q, Lc = chunk_len(j);
        const PcBuf<IO, N, P> bf = getbuf(j);
        const PcCoef co = getcoef(j);
        const bool last_chunk = j == ck1 - 1;
        const int nks = rows_pad / 32;
        const int nrb = rows_pad / 16;  // row blocks (padding rows are zero)
#pragma unroll
        for (int u = 0; u < PBW; ++u) {
          const int pb = cw + kConsWaves * u;
          if (pb >= PB) continue;
          if (has_y) {
            // carried-state operand: E^T rows p, K = n in the accumulator order
            Frag<IO> Hf[NS];
#pragma unroll
            for (int ns = 0; ns < NS; ++ns)
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                Hf[ns].set(i4, Hreg[u][2 * ns][i4]);
                Hf[ns].set(4 + i4, (2 * ns + 1 < NB) ? Hreg[u][(2 * ns + 1 < NB) ? 2 * ns + 1 : 0][i4] : 0.f);
              }
            f32x4 acc[RBM];
            float lq[RBM];
#pragma unroll
            for (int rb = 0; rb < RBM; ++rb) {
              acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
              const int tq = (16 * rb + c) >> lgR;
              lq[rb] = co.sTok[tq < Q ? tq : Q - 1].z;
            }
            // key slabs ks (rows 32ks .. 32ks+31), query row blocks rb >= 2ks;
            // loop bounds are compile-time so causal skipping costs nothing
#pragma unroll
            for (int ks = 0; ks < RBM / 2; ++ks) {
              if (ks < nks) {
                Frag<IO> Bf[2][NS];
                float kA[2][4], kB[2][4];
                int tk[2][4];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                  const int kb = 2 * ks + h2;
#pragma unroll
                  for (int ns = 0; ns < NS; ++ns) {
                    const IO* br = bf.sB + (16 * kb + c) * LDN + 32 * ns + 4 * g;
                    Bf[h2][ns].load44(br, br + 16);
                  }
#pragma unroll
                  for (int i4 = 0; i4 < 4; ++i4) {
                    tk[h2][i4] = (16 * kb + 4 * g + i4) >> lgR;
                    const float4 kt = co.sTok[tk[h2][i4] < Q ? tk[h2][i4] : Q - 1];
                    kA[h2][i4] = kt.x;
                    kB[h2][i4] = kt.y;
                  }
                }
                Frag<IO> Xf;
                {
                  const IO* xr = bf.sXt + (16 * pb + c) * ldr + 32 * ks + 4 * g;
                  Xf.load44(xr, xr + 16);
                }
#pragma unroll
                for (int rb = 2 * ks; rb < RBM; ++rb) {
                  if (rb < nrb) {
                    Frag<IO> Cf[NS];
#pragma unroll
                    for (int ns = 0; ns < NS; ++ns) {
                      const IO* cr = bf.sC + (16 * rb + c) * LDN + 32 * ns + 4 * g;
                      Cf[ns].load44(cr, cr + 16);
                    }
                    if (ks == 0) {
#pragma unroll
                      for (int ns = 0; ns < NS; ++ns) mma(acc[rb], Hf[ns], Cf[ns]);
                      acc[rb] = acc[rb] * __builtin_amdgcn_exp2f(lq[rb]);
                    }
                    const int tq = (16 * rb + c) >> lgR;
                    f32x4 St[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                      St[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
                      if (2 * ks + h2 <= rb) {
#pragma unroll
                        for (int ns = 0; ns < NS; ++ns) mma(St[h2], Bf[h2][ns], Cf[ns]);
                      }
                    }
                    Frag<IO> SM;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                      const int kb = 2 * ks + h2;
#pragma unroll
                      for (int i4 = 0; i4 < 4; ++i4) {
                        float v = 0.f;
                        if (kb <= rb) {
                          const int tkv = tk[h2][i4];
                          float m = (tkv <= tq) ? __builtin_amdgcn_exp2f(lq[rb] - kA[h2][i4]) : 0.f;
                          m += (tkv < tq) ? __builtin_amdgcn_exp2f(lq[rb] - kB[h2][i4]) : 0.f;
                          v = St[h2][i4] * m;
                          if (kb == rb) v += (4 * g + i4 == c) ? Dh : 0.f;  // skip term D x
                        }
                        SM.set(4 * h2 + i4, v);
                      }
                    }
                    mma(acc[rb], Xf, SM);
                  }
                }
              }
            }
            // store y (token t = row 16rb + c, columns 16pb + 4g .. +3)
#pragma unroll
            for (int rb = 0; rb < RBM; ++rb) {
              const int rho = 16 * rb + c;
              const int t = rho >> lgR, r = rho & (R - 1);
              if (rb < nrb && rho < rows && t < Lc) {
                const float v[4] = {acc[rb][0], acc[rb][1], acc[rb][2], acc[rb][3]};
                store4(Yg + (size_t)(c0 + t) * tokX + r * P + 16 * pb + 4 * g, v);
              }
            }
          }
          // state update and rotation into the next chunk's frame
          const float decE = expf(co.sMisc[0]);
          Frag<IO> Xs[RBM / 2];
#pragma unroll
          for (int ks = 0; ks < RBM / 2; ++ks)
            if (ks < nks) Xs[ks].load8(bf.sXt + (16 * pb + c) * ldr + 32 * ks + 8 * g);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            f32x4 hacc = Hreg[u][nb] * decE;
#pragma unroll
            for (int ks = 0; ks < RBM / 2; ++ks) {
              if (ks < nks) {
                Frag<IO> fa;
                fa.load8(bf.sBt + (16 * nb + c) * ldr + 32 * ks + 8 * g);
                mma(hacc, fa, Xs[ks]);
              }
            }
            const float4 r0 = bf.sEnd[8 * nb + 2 * g];
            const float4 r1 = bf.sEnd[8 * nb + 2 * g + 1];
            float v[4] = {hacc[0], hacc[1], hacc[2], hacc[3]};
            rot2(v[0], v[1], r0.x, r0.y);
            rot2(v[2], v[3], r1.x, r1.y);
            Hreg[u][nb] = f32x4{v[0], v[1], v[2], v[3]};
            if (last_chunk) {
              const int p = 16 * pb + c, n0 = 16 * nb + 4 * g;
              if (writes_final)
                store4(a.h + ((size_t)chain * P + p) * N + n0, v);
              else if (mode == kPcSummary)
                store4(a.seg_state + (((size_t)seg * kp.batch * H + chain) * P + p) * N + n0, v);
            }
          }
        }
        if (mode == kPcSummary) {
          const int ct = tid - kProdThreads;
          if (ct < N / 2) {
            const float tot = sSeg[ct] + bf.sEnd[ct].z;
            sSeg[ct] = tot;
            if (last_chunk) a.seg_angle[((size_t)seg * kp.batch * H + chain) * (N / 2) + ct] = tot;
          }
          if (ct == 0) {
            lsum += co.sMisc[0];
            if (last_chunk) a.seg_decay[(size_t)seg * kp.batch * H + chain] = lsum;
          }
        }
      }
      __syncthreads();
    }
  }

  if (writes_final) {
    const IO* Bl = Bg + (size_t)(T - 1) * tokBC;
    const IO* Xl = Xg + (size_t)(T - 1) * tokX;
    IO* Bp = static_cast<IO*>(a.B_prev) + (size_t)chain * R * N;
    IO* Xp = static_cast<IO*>(a.x_prev) + (size_t)chain * R * P;
    for (int e = tid; e < R * N; e += kPcThreads) Bp[e] = Bl[e];
    for (int e = tid; e < R * P; e += kPcThreads) Xp[e] = Xl[e];
  }
}

template <typename IO, int N, int P>
hipError_t launch_pc_t(const Dims& d, const PrefillArgs& a, hipStream_t st, int mode, int nblocks) {
  const int rows_pad = ((d.Q * d.R) + 31) & ~31;
  const size_t lds = PcLds<IO, N, P>::bytes(rows_pad, d.Q);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_pc_kernel<IO, N, P>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  PcParams kp;
  kp.a = a;
  kp.batch = d.batch;
  kp.heads = d.heads;
  kp.R = d.R;
  kp.lgR = d.R == 1 ? 0 : (d.R == 2 ? 1 : 2);
  kp.Q = d.Q;
  kp.mode = mode;
  kp.nblocks = nblocks;
  hipLaunchKernelGGL((prefill_pc_kernel<IO, N, P>), dim3(nblocks), dim3(kPcThreads), lds, st, kp);
  return hipGetLastError();
}

template <typename IO, int N>
hipError_t pc_p(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nb) {
  switch (d.P) {
    case 16: return launch_pc_t<IO, N, 16>(d, a, s, mode, nb);
    case 32: return launch_pc_t<IO, N, 32>(d, a, s, mode, nb);
    case 64: return launch_pc_t<IO, N, 64>(d, a, s, mode, nb);
    default: return launch_pc_t<IO, N, 128>(d, a, s, mode, nb);
  }
}

template <typename IO>
hipError_t pc_n(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nb) {
  switch (d.N) {
    case 16: return pc_p<IO, 16>(d, a, s, mode, nb);
    case 32: return pc_p<IO, 32>(d, a, s, mode, nb);
    case 64: return pc_p<IO, 64>(d, a, s, mode, nb);
    default: return pc_p<IO, 128>(d, a, s, mode, nb);
  }
}

template <typename IO>
int pc_max_rows(const Dims& d) {
  switch (d.N * 1000 + d.P) {
#define M3_CASE(NN, PP) \
  case NN * 1000 + PP: return PcLimits<IO, NN, PP>::kMaxRows;
    M3_CASE(16, 16) M3_CASE(16, 32) M3_CASE(16, 64) M3_CASE(16, 128)
    M3_CASE(32, 16) M3_CASE(32, 32) M3_CASE(32, 64) M3_CASE(32, 128)
    M3_CASE(64, 16) M3_CASE(64, 32) M3_CASE(64, 64) M3_CASE(64, 128)
    M3_CASE(128, 16) M3_CASE(128, 32) M3_CASE(128, 64) M3_CASE(128, 128)
#undef M3_CASE
    default: return 0;
  }
}

}  // namespace

bool prefill_pc_supported(const Dims& d) {
  const int rows_pad = ((d.Q * d.R) + 31) & ~31;
  return rows_pad <= (d.bf16 ? pc_max_rows<bf16>(d) : pc_max_rows<float>(d));
}

hipError_t launch_prefill_pc(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks) {
  return d.bf16 ? pc_n<bf16>(d, a, s, mode, nblocks) : pc_n<float>(d, a, s, mode, nblocks);
}

}  // namespace m3
