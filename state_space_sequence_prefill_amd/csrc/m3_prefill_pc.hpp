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
// Included by m3_prefill_pc.hip (plain y store), m3_prefill_pc_gated.hip (y
// through the output epilogue) and m3_prefill_pc_down.hip (the MIMO rank
// down-projection, then the epilogue), one set of instances each.
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
//     y^T into an LDS output tile, which leaves for HBM as whole rows at the
//     start of the next chunk.
// Two workgroup barriers per chunk separate the roles' buffers: tiles are
// double buffered, per-token coefficients triple buffered (written one chunk
// ahead by the producers, read by producers in the next chunk and by
// consumers in the one after).
#pragma once

#include "m3_kernels.hpp"
#include "m3_mfma.hpp"

namespace m3 {
namespace {

constexpr int kPcThreads = 512;
constexpr int kProdThreads = 256;
constexpr int kConsWaves = 4;
constexpr float kLog2ePc = 1.4426950408889634f;

enum PcMode : int { kPcFused = 0, kPcSummary = 1, kPcSegment = 2 };

// R is the rank of the data; the tiles hold 2^lgR >= R rows per token (the
// rank padded to a power of two: rows of the padded ranks carry x = 0, so
// they add nothing, and their outputs are not stored).
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

// LDS layout for <IO, N, P> with tiles of `rows` (token, rank) rows; BCN
// adds the BC normalisation's weights and partial sums of squares.
template <typename IO, int N, int P, bool BCN = false>
struct PcLds {
  static constexpr int E = sizeof(IO);
  static constexpr int PAD = 16 / E;
  static constexpr int NK = N < 32 ? 32 : N;
  static constexpr int LDN = NK + PAD;
  // one tile buffer
  __host__ __device__ static constexpr size_t buf_bytes(int rows) {
    return (size_t)rows * LDN * E * 2            // sB, sC
           + (size_t)N * (rows + PAD) * E        // sBt
           + (size_t)P * (rows + PAD) * E        // sXt
           + (size_t)(N / 2) * 16;               // sEnd: {cos, sin} of pair pairs, then the angles
  }
  // masked score tile (S.M) shared by the consumer waves: rows = queries,
  // columns = keys
  __host__ __device__ static constexpr size_t sm_bytes(int rows) { return (size_t)rows * (rows + PAD) * E; }
  // output tile: the consumer waves' y slices meet here and leave as whole rows
  __host__ __device__ static constexpr size_t y_bytes(int rows) { return (size_t)rows * (P + PAD) * E; }
  static constexpr size_t kCoefBytes = 64 * 20 + 16;  // one coefficient slot (Q <= 64)
  // BC normalisation: a row's N columns are spread over norm_groups(rows)
  // producer lane groups, whose partial sums of squares meet here
  // ([B, C][group][rows]), after the weights of B and C (2 N floats)
  __host__ __device__ static constexpr int norm_groups(int rows) {
    return (N / 8) * rows / 256 > 1 ? (N / 8) * rows / 256 : 1;
  }
  __host__ __device__ static constexpr size_t norm_bytes(int rows) {
    return BCN ? (size_t)2 * N * 4 + (size_t)2 * norm_groups(rows) * rows * 4 : 0;
  }
  __host__ __device__ static constexpr size_t bytes(int rows) {
    return 2 * buf_bytes(rows) + sm_bytes(rows) + y_bytes(rows) + 3 * kCoefBytes + (N / 2) * 4 + norm_bytes(rows);
  }
};

template <typename IO, int N, int P>
struct PcBuf {
  IO *sB, *sC, *sBt, *sXt;
  // end rotations: float4 q = {cos, sin} of pairs 2q and 2q + 1 (q < N/4),
  // then the N/2 angles as floats (float4 N/4 on)
  float4* sEnd;
};
struct PcCoef {
  float4* sTok;  // [Q] {A_t, B_t, L_t, Kf_t}: mask exponents, log2-decay, key factor
  float* sW;     // [Q] state-update weights
  float* sMisc;  // [0] l_E, [1] l_E*log2e
};

// Largest padded row count and register-array bounds of an instance.
template <typename IO, int N, int P>
struct PcLimits {
  static constexpr int NK = PcLds<IO, N, P>::NK;
  static constexpr bool fits(int r) {
    return PcLds<IO, N, P>::bytes(r) <= 160 * 1024 && r * NK * (int)sizeof(IO) <= 16384 &&
           (r / 4) * (N / 8) <= 2 * kProdThreads && (r / 4) * (P / 8) <= 2 * kProdThreads;
  }
  static constexpr int kMaxRows = fits(128) ? 128 : fits(64) ? 64 : fits(32) ? 32 : 0;
  static constexpr int kMaxRB = kMaxRows / 16;                                    // row blocks
  static constexpr int kMI = (kMaxRows / 4) * (N / 8) > kProdThreads ? 2 : 1;     // B/C items per thread
  static constexpr int kMX = (kMaxRows / 4) * (P / 8) > kProdThreads ? 2 : 1;     // x items per thread
  static constexpr int kPBW = (P / 16 + kConsWaves - 1) / kConsWaves;            // p-blocks per consumer
};

// One chunk's raw inputs as a producer thread holds them in registers.
template <typename IO, int MI, int MX>
struct PcRaw {
  Raw8<IO> b[MI][4], c[MI][4], x[MX][4];
  float4 th[MI][4];
};

// How y leaves the kernel.
enum PcEpi : int {
  kEpiPlain = 0,  // the scan output (batch, T, H, R, P)
  kEpiGate = 1,   // pre-gate grouped RMSNorm per (token, head, rank) row (a.gz, a.gw, a.geps)
  kEpiDown = 2,   // rank down-projection (a.gdown) to (batch, T, H, P), then the same epilogue per (token, head)
};

// BCN: B and C rows are RMS-normalised and scaled per channel (a.nbw, a.ncw,
// a.neps) as the producers build the tiles; the pending B_prev of the entry
// state likewise.
// LGR >= 0 fixes log2 of the padded rank at compile time (0: rank 1; 2:
// ranks 3 and 4), and except with the gated per-rank epilogue also the tile
// height at the largest that fits (kMaxRows rows, kMaxRows >> LGR tokens; such an instance
// is launched only for calls at that height), so the row -> (token, rank)
// arithmetic and the chunk-sized bounds fold away.  -1 takes both from kp.
// SUMM fixes the segment-summary mode: no C loads, scores, outputs or y.
template <typename IO, int N, int P, int EPI, bool BCN, int LGR, bool SUMM = false>
__global__ __launch_bounds__(kPcThreads, 1) void prefill_pc_kernel(PcParams kp) {
  using L = PcLds<IO, N, P, BCN>;
  using Lim = PcLimits<IO, N, P>;
  constexpr int NB = N / 16, PB = P / 16;
  constexpr int NK = L::NK, LDN = L::LDN, PAD = L::PAD;
  constexpr int NS = NK / 32;
  constexpr int MI = Lim::kMI, MX = Lim::kMX, PBW = Lim::kPBW;
  // Split producer roles when a chunk holds at most half as many B/C items
  // (and x items) as there are producer threads: waves 0-1 then take the B
  // rows of the items (B~, its weighted tile, the end rotations), waves 2-3
  // the C rows and x, so each thread rotates one matrix instead of two and no
  // wave works on duplicates only.
  constexpr bool kSplit = (Lim::kMaxRows / 4) * (N / 8) <= kProdThreads / 2 &&
                          (Lim::kMaxRows / 4) * (P / 8) <= kProdThreads / 2;
  // Tiles always hold RMAX rows; rows past Q*R stay zero, so every consumer
  // loop has compile-time bounds.
  // (instances whose tiles do not fit at all are never launched; they compile
  // with the smallest tile height)
  constexpr int RMAX = Lim::kMaxRows > 0 ? Lim::kMaxRows : 32, KSM = RMAX / 32, RBM = RMAX / 16;
  constexpr int ldr = RMAX + PAD;
  extern __shared__ __align__(16) char smem[];

  const PrefillArgs& a = kp.a;
  const int Q = (LGR >= 0 && EPI != kEpiGate) ? (Lim::kMaxRows > 0 ? Lim::kMaxRows : 32) >> LGR : kp.Q;
  const int R = LGR == 0 ? 1 : kp.R, lgR = LGR >= 0 ? LGR : kp.lgR, H = kp.heads;
  const int RP = 1 << lgR;  // tile rows per token (R padded to a power of two)
  const int T = a.seqlen;
  const int mode = SUMM ? (int)kPcSummary : kp.mode;
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
  const int rows = Q * RP;
  const int rows_pad = (rows + 31) & ~31;

  // ---- LDS: [tile buffer 0 | tile buffer 1 | sSM | sY | coefs x3 | sSeg] ----
  constexpr size_t bufB = (size_t)RMAX * LDN * sizeof(IO);  // sB, sC
  constexpr size_t bufBt = (size_t)N * ldr * sizeof(IO);
  constexpr size_t bufXt = (size_t)P * ldr * sizeof(IO);
  constexpr size_t bufStride = L::buf_bytes(RMAX);
  constexpr size_t coefStride = L::kCoefBytes;
  constexpr size_t smStride = L::sm_bytes(RMAX);
  constexpr size_t yStride = L::y_bytes(RMAX);
  constexpr int ldy = P + PAD;
  IO* const sSM = reinterpret_cast<IO*>(smem + 2 * bufStride);
  IO* const sY = reinterpret_cast<IO*>(smem + 2 * bufStride + smStride);
  char* const coefBase = smem + 2 * bufStride + smStride + yStride;
  float* const sSeg = reinterpret_cast<float*>(coefBase + 3 * coefStride);
  float* const sGw = sSeg + N / 2;         // BCN: weights of B (N) and C (N)
  float* const sPart = sGw + 2 * N;        // BCN: [B, C][group][rows_pad] partial sums
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
  // Zero both tile buffers and the score tile once: padding rows and
  // columns, and score blocks above the diagonal, are never written.
  for (size_t e = tid; e < (2 * bufStride + smStride) / 16; e += kPcThreads)
    reinterpret_cast<uint4*>(smem)[e] = make_uint4(0u, 0u, 0u, 0u);
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
    // 4 state pairs = 8 columns).  Lanes run over GW adjacent pair groups
    // first, then over the RG = rows_pad/4 row groups, so 16 lanes read GW*16
    // contiguous bytes of 16/GW rows (few cache lines per load instruction),
    // and the RG row groups of one pair group stay inside one wave (GW*RG <=
    // 64): the angle prefix over the chunk is an in-wave strided scan.
    // Inside the chunk loop every load and every use of a loaded register is
    // unconditional (threads past the item count work on a clamped duplicate
    // item and skip only their LDS stores): a load or use behind a branch
    // would make the compiler wait for all outstanding loads.
    const int pt = tid;
    const int pw = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform producer index
    const bool crole = kSplit && pw >= 2;                 // split roles: this thread's rows are C's
    const int RG = rows_pad / 4;
    const int npg = N / 8;
    const int GW = npg < 64 / RG ? npg : 64 / RG;  // pair groups per lane group
    const int npx = P / 8;
    const int GX = npx < 64 / RG ? npx : 64 / RG;  // x column groups per lane group
    const int nbitems = RG * npg;
    const int nxitems = RG * npx;
    // tokens per row group: 4 / RP, or with RP = 8 half a token (the even
    // row group of a token carries its angle, the odd one none)
    const int ntok = lgR <= 2 ? 4 >> lgR : 1;
    const IO* const Csrc = has_y ? Cg : Bg;  // segment summaries never read C
    // Two register sets: chunk i is built from one while chunk i+1's loads
    // land in the other, and chunk i+2's loads are issued into the first
    // right after it is consumed (two chunks of HBM latency hidden).
    PcRaw<IO, MI, MX> rsA, rsB;
    float rdt, rlm, rdtn, rlmn;  // raw dt/lam of the chunk after next

    // Per item: row group, column group, and 32-bit element offsets of its
    // rows relative to the chunk's first token (the host keeps
    // chunk * heads * rank * max(N, P) below 2^31).
    int irg[MI], ipg[MI], rtok[MI][4];
    bool ist[MI];
    uint32_t ob[MI][4], oth[MI][4], obs[MI], oths[MI];
    int xrg[MX], xxg[MX], xtok[MX][4];
    bool xst[MX], xpad[MX][4];  // xpad: a padded rank's row (its x is zero)
    uint32_t ox[MX][4], oxs[MX];
#pragma unroll
    for (int m = 0; m < MI; ++m) {
      const int it0 = (kSplit ? pt & (kProdThreads / 2 - 1) : pt) + m * kProdThreads;
      ist[m] = it0 < nbitems;
      const int it = ist[m] ? it0 : it0 % nbitems;
      const int rg = (it / GW) % RG, pg = (it / (GW * RG)) * GW + it % GW;
      irg[m] = rg;
      ipg[m] = pg;
      const int t0 = (4 * rg) >> lgR;
      obs[m] = 8u * pg;
      oths[m] = 4u * pg;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rho = 4 * rg + k;
        rtok[m][k] = rho < rows ? (rho >> lgR) : Q;
        const int rk = (rho & (RP - 1)) < R ? (rho & (RP - 1)) : R - 1;  // padded ranks read a real row
        ob[m][k] = (uint32_t)(rho >> lgR) * (uint32_t)tokBC + (uint32_t)rk * N + 8 * pg;
        oth[m][k] = (uint32_t)(t0 + (k < ntok ? k : ntok - 1)) * (uint32_t)tokTh + 4 * pg;
      }
    }
#pragma unroll
    for (int m = 0; m < MX; ++m) {
      const int it0 = (kSplit ? pt ^ (kProdThreads / 2) : pt) + m * kProdThreads;  // split: waves 2-3
      xst[m] = it0 < nxitems;
      const int it = xst[m] ? it0 : it0 % nxitems;
      const int rg = (it / GX) % RG, xg = (it / (GX * RG)) * GX + it % GX;
      xrg[m] = rg;
      xxg[m] = xg;
      oxs[m] = 8u * xg;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rho = 4 * rg + k;
        xtok[m][k] = rho < rows ? (rho >> lgR) : Q;
        xpad[m][k] = (rho & (RP - 1)) >= R;
        const int rk = xpad[m][k] ? R - 1 : (rho & (RP - 1));
        ox[m][k] = (uint32_t)(rho >> lgR) * (uint32_t)tokX + (uint32_t)rk * P + 8 * xg;
      }
    }

    auto load_chunk = [&](int ck, PcRaw<IO, MI, MX>& rs) {  // B, C, x, theta of chunk ck (rows past the chunk read token 0)
      const int c0 = ck * Q, Lc = chunk_len(ck);
      const IO* Bc = Bg + (size_t)c0 * tokBC;
      const IO* Cc = Csrc + (size_t)c0 * tokBC;
      const IO* Xc = Xg + (size_t)c0 * tokX;
      const float* Tc = THg + (size_t)c0 * tokTh;
#pragma unroll
      for (int m = 0; m < MI; ++m) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t o = rtok[m][k] < Lc ? ob[m][k] : obs[m];
          if constexpr (kSplit) {
            rs.b[m][k].load((crole ? Cc : Bc) + o);  // this role's matrix
          } else {
            rs.b[m][k].load(Bc + o);
            if constexpr (!SUMM) rs.c[m][k].load(Cc + o);  // (a summary reads no C)
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t o = rtok[m][0] + (q < ntok ? q : ntok - 1) < Lc ? oth[m][q] : oths[m];
          rs.th[m][q] = *reinterpret_cast<const float4*>(Tc + o);
        }
      }
#pragma unroll
      for (int m = 0; m < MX; ++m) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t o = xtok[m][k] < Lc ? ox[m][k] : oxs[m];
          rs.x[m][k].load(Xc + o);
        }
      }
    };
    // BC normalisation, first half: the sums of squares of this thread's row
    // pieces of the chunk held in `rs`, summed over the GW lanes that share
    // the rows, into sPart (one float4 of 4 rows per lane group).  The other
    // half reads them back while building the chunk's tiles.
    // (GW <= 8: rows_pad >= 32 gives RG >= 8; the sums take no branches)
    const int NG = npg / GW;  // lane groups per row
    constexpr int kGWMax = (N / 8) < 8 ? (N / 8) : 8;
    auto norm_partials = [&](const PcRaw<IO, MI, MX>& rs) {
      if constexpr (BCN) {
#pragma unroll
        for (int m = 0; m < MI; ++m) {
          float pb[4], pc[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            pb[k] = lane_group_sum_upto<kGWMax>(rs.b[m][k].sumsq(), GW);
            // (a segment summary holds B in the C registers and uses no C sums)
            pc[k] = (kSplit || SUMM) ? 0.f : lane_group_sum_upto<kGWMax>(rs.c[m][k].sumsq(), GW);
          }
          if (kSplit && ist[m] && (lane & (GW - 1)) == 0) {  // this role's matrix only
            const int grp = ipg[m] / GW + (crole ? NG : 0);
            *reinterpret_cast<float4*>(sPart + (size_t)grp * rows_pad + 4 * irg[m]) =
                make_float4(pb[0], pb[1], pb[2], pb[3]);
          }
          if (!kSplit && ist[m] && (lane & (GW - 1)) == 0) {
            const int grp = ipg[m] / GW;
            *reinterpret_cast<float4*>(sPart + (size_t)grp * rows_pad + 4 * irg[m]) =
                make_float4(pb[0], pb[1], pb[2], pb[3]);
            *reinterpret_cast<float4*>(sPart + (size_t)(NG + grp) * rows_pad + 4 * irg[m]) =
                make_float4(pc[0], pc[1], pc[2], pc[3]);
          }
        }
      }
    };
    auto load_dt = [&](int ck) {  // dt, lam of chunk ck (lane = token) and of the token after it
      const int c0 = ck * Q, Lc = chunk_len(ck);
      const int t = lane < Lc ? lane : Lc - 1;
      rdt = DTg[(size_t)(c0 + t) * H];
      rlm = LMg[(size_t)(c0 + t) * H];
      const int tn = (c0 + Lc < T) ? c0 + Lc : c0 + Lc - 1;
      rdtn = DTg[(size_t)tn * H];
      rlmn = LMg[(size_t)tn * H];
    };
    // In-chunk decay scan and per-token coefficients of chunk ck -> coef slot
    // ck % 3 (producer wave 0 only, which alone loads dt and lam).
    // sTok[t] = {A_t, B_t, L_t, Kf_t} with L_t = l_t log2(e) and the mask weights
    // gamma_t 2^{L_q - L_t} = 2^{L_q - A_t},  beta_{t+1} 2^{L_q - L_{t+1}} = 2^{L_q - B_t}
    // (a zero weight gives an infinite exponent and an exact zero).
    auto decay_coefs = [&](int ck, bool store) {
      const int c0 = ck * Q, Lc = chunk_len(ck);
      const bool fold_next = c0 + Lc < T;
      const PcCoef co = getcoef(ck);
      const int t = lane;
      const bool valid = t < Lc;
      const float dtv = valid ? rdt : 0.f, lmv = valid ? rlm : 0.f;
      const float av = (valid && t > 0) ? log_decay(dtv, Ah) : 0.f;
      const float ell = wave_inclusive_scan(av);
      const float2 wt = input_weights(dtv, lmv, expf(dtv * Ah), a.disc);
      const float bet = wt.x, gam = wt.y;
      const float dtn = fold_next ? rdtn : 0.f, lmn = fold_next ? rlmn : 0.f;
      const float ell_last = __shfl(ell, Lc - 1, kWave);
      const float ellE = ell_last + log_decay(dtn, Ah);
      const float bet_up = __shfl_down(bet, 1, kWave);
      const float ell_up = __shfl_down(ell, 1, kWave);
      const bool inner = t < Lc - 1, lastv = t == Lc - 1;
      const float betn = inner ? bet_up : (lastv ? input_weights(dtn, lmn, expf(dtn * Ah), a.disc).x : 0.f);
      const float elln = inner ? ell_up : ellE;
      const float ellv = valid ? ell : ell_last;
      const float w = valid ? (gam * expf(ellE - ellv) + betn * expf(ellE - elln)) : 0.f;
      const float inf = __builtin_huge_valf();
      const float L2 = ellv * kLog2ePc;
      const float Ak = (valid && gam > 0.f) ? L2 - __log2f(gam) : inf;
      const float Bk = (valid && betn > 0.f) ? elln * kLog2ePc - __log2f(betn) : inf;
      // key factor for score blocks below the diagonal: with e the last token
      // of the key's 16-row block, every query q of a later block has q >=
      // e + 1, and M[q][k] = 2^{L_q - L_{e+1}} * Kf_k with
      //   Kf_k = gamma_k 2^{L_{e+1} - L_k} + beta_{k+1} 2^{L_{e+1} - L_{k+1}}.
      // Both exponents of Kf and the row factor's are <= 0 (the log-decays
      // only fall), so neither factor overflows for any decay: Kf_k <=
      // gamma_k + beta_{k+1}, and the row factor <= 1.  When e + 1 is past
      // the chunk no valid query uses Kf, and L_E keeps it bounded.
      const int te1 = (t | ((16 >> lgR) - 1)) + 1;
      const float Le1s = __shfl(L2, te1 < Lc ? te1 : Lc - 1, kWave);
      const float Le1 = te1 < Lc ? Le1s : ellE * kLog2ePc;
      const float Kf = valid ? gam * exp2f(Le1 - L2) + betn * exp2f(Le1 - elln * kLog2ePc) : 0.f;
      if (store && t < Q) {
        co.sTok[t] = make_float4(Ak, Bk, L2, Kf);
        co.sW[t] = w;
        if (t == 0) {
          co.sMisc[0] = ellE;
          co.sMisc[1] = ellE * kLog2ePc;
        }
      }
    };
    // Angles (in-wave scan), rotation, and the tiles of chunk ck -> tile buffer ck % 2.
    auto build_tiles = [&](int ck, const PcRaw<IO, MI, MX>& rs) {
      const int Lc = chunk_len(ck);
      const int te = Lc - 1;
      const PcBuf<IO, N, P> bf = getbuf(ck);
      const float* sW = getcoef(ck).sW;
#pragma unroll
      for (int m = 0; m < MI; ++m) {
        const int rg = irg[m], pg = ipg[m];
        const int t0 = rtok[m][0];
        float th[4][4];
        const int ntk = (lgR == 3 && (rg & 1)) ? 0 : ntok;  // RP = 8: odd row groups add no angle
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float tv = (q < ntk && t0 + q < Lc) ? 1.f : 0.f;
          th[q][0] = tv * rs.th[m][q].x;
          th[q][1] = tv * rs.th[m][q].y;
          th[q][2] = tv * rs.th[m][q].z;
          th[q][3] = tv * rs.th[m][q].w;
          if constexpr (sizeof(IO) == 4) {  // fp32: keep the angle sums small (bf16's hardware trig reduces them)
#pragma unroll
            for (int j = 0; j < 4; ++j) th[q][j] = reduce_angle(th[q][j]);
          }
        }
        // exclusive prefix of the row groups' totals within the pair group
        float base[4], tot[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tot[j] = th[0][j] + th[1][j] + th[2][j] + th[3][j];
          base[j] = tot[j];
        }
        strided_inclusive_scan(base, GW, RG);
#pragma unroll
        for (int j = 0; j < 4; ++j) base[j] -= tot[j];
        // per-row angles: rows of one token share its prefix
        float ph[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int kq = k >> lgR;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            ph[k][j] = base[j] + th[0][j] + (kq >= 1 ? th[1][j] : 0.f) + (kq >= 2 ? th[2][j] : 0.f) +
                       (kq >= 3 ? th[3][j] : 0.f);
        }
        // BC normalisation, second half: this item's 4 row scales and 8
        // column weights of B and C.  The GW lanes that share the item's rows
        // split the NG group partials between them (lane j reads groups j,
        // j + GW, ...: one LDS round trip instead of NG) and sum the rest
        // across the lanes.
        float sclB[4] = {1.f, 1.f, 1.f, 1.f}, sclC[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (BCN) {
          float4 tb = make_float4(0.f, 0.f, 0.f, 0.f), tc = tb;
          for (int grp = lane & (GW - 1); grp < NG; grp += GW) {
            if (kSplit) {  // this role's rows
              const float4 u =
                  *reinterpret_cast<const float4*>(sPart + (size_t)(grp + (crole ? NG : 0)) * rows_pad + 4 * rg);
              tb.x += u.x; tb.y += u.y; tb.z += u.z; tb.w += u.w;
              continue;
            }
            const float4 u = *reinterpret_cast<const float4*>(sPart + (size_t)grp * rows_pad + 4 * rg);
            const float4 w = *reinterpret_cast<const float4*>(sPart + (size_t)(NG + grp) * rows_pad + 4 * rg);
            tb.x += u.x; tb.y += u.y; tb.z += u.z; tb.w += u.w;
            tc.x += w.x; tc.y += w.y; tc.z += w.z; tc.w += w.w;
          }
          tb.x = lane_group_sum_upto<kGWMax>(tb.x, GW); tb.y = lane_group_sum_upto<kGWMax>(tb.y, GW);
          tb.z = lane_group_sum_upto<kGWMax>(tb.z, GW); tb.w = lane_group_sum_upto<kGWMax>(tb.w, GW);
          if (!kSplit) {
            tc.x = lane_group_sum_upto<kGWMax>(tc.x, GW); tc.y = lane_group_sum_upto<kGWMax>(tc.y, GW);
            tc.z = lane_group_sum_upto<kGWMax>(tc.z, GW); tc.w = lane_group_sum_upto<kGWMax>(tc.w, GW);
          }
          const float inN = 1.0f / N;
          sclB[0] = rsqrtf(tb.x * inN + a.neps); sclB[1] = rsqrtf(tb.y * inN + a.neps);
          sclB[2] = rsqrtf(tb.z * inN + a.neps); sclB[3] = rsqrtf(tb.w * inN + a.neps);
          sclC[0] = rsqrtf(tc.x * inN + a.neps); sclC[1] = rsqrtf(tc.y * inN + a.neps);
          sclC[2] = rsqrtf(tc.z * inN + a.neps); sclC[3] = rsqrtf(tc.w * inN + a.neps);
        }
        float bt[4][8];
        float cs4[4], sn4[4];  // sines and cosines of the current row's token
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int rho = 4 * rg + k;
          const int t = rtok[m][k];
          // rows past the chunk hold finite duplicates (clamped loads); every
          // use of them is weighted by an exact zero (mask, w) or never stored
          const bool valid = t < Lc;
          float bv[8];
          rs.b[m][k].unpack(bv);
          if constexpr (BCN) {  // column weights read where used (registers are scarce here)
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[e] *= sGw[(crole ? N : 0) + 8 * pg + e] * sclB[k];
          }
          // rows of one token share its angles: with RP rows per token only
          // the first row of each token evaluates them (a uniform branch)
          if ((k & (RP - 1)) == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) trig<IO>(ph[k][j], sn4[j], cs4[j]);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) rot2(bv[2 * j], bv[2 * j + 1], cs4[j], -sn4[j]);
          const float wt = valid ? sW[t < Q ? t : 0] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) bt[k][e] = bv[e] * wt;
          // the row-major B~ and C~ tiles feed only the outputs; a segment
          // summary needs just the state update's tiles
          if (kSplit && ist[m] && has_y) store8((crole ? bf.sC : bf.sB) + rho * LDN + 8 * pg, bv);
          if (!kSplit && ist[m] && has_y) {
            float cv[8];
            rs.c[m][k].unpack(cv);
            if constexpr (BCN) {
#pragma unroll
              for (int e = 0; e < 8; ++e) cv[e] *= sGw[N + 8 * pg + e] * sclC[k];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) rot2(cv[2 * j], cv[2 * j + 1], cs4[j], -sn4[j]);
            store8(bf.sB + rho * LDN + 8 * pg, bv);
            store8(bf.sC + rho * LDN + 8 * pg, cv);
          }
          if (ist[m] && !crole) {
            if (valid && t == te && (rho & (RP - 1)) == 0) {
              bf.sEnd[2 * pg] = make_float4(cs4[0], sn4[0], cs4[1], sn4[1]);
              bf.sEnd[2 * pg + 1] = make_float4(cs4[2], sn4[2], cs4[3], sn4[3]);
              bf.sEnd[N / 4 + pg] = make_float4(ph[k][0], ph[k][1], ph[k][2], ph[k][3]);
            }
          }
        }
        if (ist[m] && !crole) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float col[4] = {bt[0][e], bt[1][e], bt[2][e], bt[3][e]};
            store4(bf.sBt + (8 * pg + e) * ldr + 4 * rg, col);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MX; ++m) {
        const int rg = xrg[m], xg = xxg[m];
        if constexpr (sizeof(IO) == 2) {
          // transpose 4 rows x 8 bf16 columns with byte permutes (no unpack)
          uint32_t w[4][4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) w[k][q] = rs.x[m][k].w[q];
          if (R != RP) {  // padded ranks: their rows of X^T are zero
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
              for (int q = 0; q < 4; ++q) w[k][q] = xpad[m][k] ? 0u : w[k][q];
          }
          uint2 v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            v[e].x = __builtin_amdgcn_perm(w[1][e >> 1], w[0][e >> 1], sel);
            v[e].y = __builtin_amdgcn_perm(w[3][e >> 1], w[2][e >> 1], sel);
          }
          if (xst[m]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) *reinterpret_cast<uint2*>(bf.sXt + (8 * xg + e) * ldr + 4 * rg) = v[e];
          }
        } else {
          float xv[4][8];
#pragma unroll
          for (int k = 0; k < 4; ++k) rs.x[m][k].unpack(xv[k]);
          if (R != RP) {  // padded ranks: their rows of X^T are zero
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
              for (int e = 0; e < 8; ++e) xv[k][e] = xpad[m][k] ? 0.f : xv[k][e];
          }
          if (xst[m]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float col[4] = {xv[0][e], xv[1][e], xv[2][e], xv[3][e]};
              store4(bf.sXt + (8 * xg + e) * ldr + 4 * rg, col);
            }
          }
        }
      }
    };

    // One pipeline step = one chunk and two barriers (the consumers count the
    // same: two per chunk plus a last pair).  Building chunk i overlaps the
    // consumers' shared score tile of chunk i-1 (other buffers); the first
    // barrier ends both, and the coefficient work and the next loads then
    // overlap the consumers' outputs and state update.
    // Wave priorities (issue arbitration on a SIMD, where one producer and
    // one consumer wave share the issue slots): the tile build is the longer
    // side of the first phase, so it runs at raised priority.
    auto step = [&](int i, PcRaw<IO, MI, MX>& rs, const PcRaw<IO, MI, MX>& rsn) {
      __builtin_amdgcn_s_setprio(2);
      build_tiles(i, rs);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      const int n1 = i + 1 < ck1 ? i + 1 : i;  // clamped: past the end the data is reloaded, not used
      const int n2 = i + 2 < ck1 ? i + 2 : n1;
      if (pw == 0) {
        decay_coefs(n1, n1 != i);
        // dt first: the vmcnt counter is in order, so consuming dt next step
        // then leaves this step's chunk batch in flight
        load_dt(n2);
      }
      load_chunk(n2, rs);
      // BCN: row sums of the next chunk (its loads were issued a step ago;
      // the in-order counter leaves the loads just issued in flight)
      norm_partials(rsn);
      __syncthreads();
    };
    if constexpr (BCN) {
      for (int j = pt; j < 2 * N; j += kProdThreads)
        sGw[j] = j < N ? a.nbw[(size_t)hh * N + j] : a.ncw[(size_t)hh * N + j - N];
    }
    // bf16 I/O keeps two chunks of raw inputs in flight; fp32 I/O, whose raw
    // chunk takes twice the registers, one (loaded right after the tiles of
    // the previous one are built, so it arrives during the consumers' phase)
    constexpr bool kTwoAhead = sizeof(IO) == 2;
    if (ck0 < ck1) {
      // prologue: coefficients of the first chunk, then the first prefetches
      const int n1 = ck0 + 1 < ck1 ? ck0 + 1 : ck0;
      if (pw == 0) {
        load_dt(ck0);
        decay_coefs(ck0, true);
      }
      load_chunk(ck0, rsA);
      if (pw == 0) load_dt(n1);
      if constexpr (kTwoAhead) load_chunk(n1, rsB);
      norm_partials(rsA);
    }
    __syncthreads();
    if constexpr (kTwoAhead) {
      // the pair loop has no conditional loads, so the wait counts the compiler
      // derives around its back edge stay exact (only the batch consumed waits)
      int i = ck0;
      for (; i + 1 < ck1; i += 2) {
        step(i, rsA, rsB);
        step(i + 1, rsB, rsA);
      }
      if (i < ck1) step(i, rsA, rsB);
    } else {
      for (int i = ck0; i < ck1; ++i) {
        __builtin_amdgcn_s_setprio(2);
        build_tiles(i, rsA);
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        const int n1 = i + 1 < ck1 ? i + 1 : i;
        const int n2 = i + 2 < ck1 ? i + 2 : n1;
        if (pw == 0) {
          decay_coefs(n1, n1 != i);
          load_dt(n2);
        }
        load_chunk(n1, rsA);
        norm_partials(rsA);
        __syncthreads();
      }
    }
    __syncthreads();
    __syncthreads();
  } else {
    // ======================= consumers (waves 4-7) =======================
    const int cw = __builtin_amdgcn_readfirstlane(wave - 4);  // wave-uniform
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
        beta0 = input_weights(dt0, lm0, alpha0, a.disc).x;
      }
      // BCN: RMS scales of the pending B_prev rows (lane (g, c) sums its
      // columns 16 nb + 4 g + i; the four g lanes complete the row)
      float bsc[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
      if constexpr (BCN) {
        if (mode == kPcFused) {
          const IO* Bp = static_cast<const IO*>(a.B_prev) + (size_t)chain * R * N;
#pragma unroll
          for (int r = 0; r < 8; ++r) {  // R <= 8
            if (r < R) {
              float ss = 0.f;
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) {
                float bp[4];
                load4(Bp + r * N + 16 * nb + 4 * g, bp);
                ss += bp[0] * bp[0] + bp[1] * bp[1] + bp[2] * bp[2] + bp[3] * bp[3];
              }
              ss += shfl_xor(ss, 16);
              ss += shfl_xor(ss, 32);
              bsc[r] = rsqrtf(ss * (1.0f / N) + a.neps);
            }
          }
        }
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
#pragma unroll
              for (int r = 0; r < 8; ++r) {  // R <= 8
                if (r < R) {
                  float bp[4];
                  load4(Bp + r * N + n0, bp);
                  const float xp = beta0 * to_f32(Xp[r * P + p]) * bsc[r];
#pragma unroll
                  for (int i4 = 0; i4 < 4; ++i4)
                    v[i4] += xp * bp[i4] * (BCN ? a.nbw[(size_t)hh * N + n0 + i4] : 1.f);
                }
              }
            } else if (mode == kPcSegment) {
              load4(a.seg_state + (((size_t)seg * kp.batch * H + chain) * P + p) * N + n0, v);
            }
            Hreg[u][nb] = f32x4{v[0], v[1], v[2], v[3]};
          }
        }
      }
    }
    // Gated: the entry-state loads retire here, once; otherwise the loop below
    // waits for every outstanding memory operation (the gate loads of the
    // next chunk among them) at each first use of Hreg.  Measured: 2% faster
    // with the epilogue, and 1% slower without it, where no load is in flight.
    if constexpr (EPI != kEpiPlain) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    // y of chunk jy leaves the LDS output tile as whole 16-byte runs of its
    // rows (each (token, rank) row is P contiguous elements in HBM)
    constexpr int EG = Gran<IO>::kN;                 // elements per 16-byte granule
    constexpr int G16 = P / EG;                      // granules per row (2 .. 32)
    constexpr int kCT = kConsWaves * kWave;          // consumer threads
    constexpr int KZ = (RMAX * G16 + kCT - 1) / kCT;  // granules per consumer thread
    const int ct = tid - kProdThreads;
    // output-tile row -> (token, rank); rows of padded ranks map to rank R-1
    // (read as clamped duplicates, never stored)
    auto rank_of = [&](int row) { return (row & (RP - 1)) < R ? (row & (RP - 1)) : R - 1; };
    auto real_row = [&](int row) { return (row & (RP - 1)) < R; };
    auto gran_off = [&](int c0, int e) -> size_t {
      const int row = e / G16, gq = e % G16;
      return (size_t)(c0 + (row >> lgR)) * tokX + rank_of(row) * P + gq * EG;
    };
    // Output epilogue (pre-gate grouped RMSNorm): a consumer thread always
    // handles granule column ct % G16 of its rows (kCT is a multiple of G16),
    // so its EG weights are loaded once; the G16 granules of one row sit in
    // G16 aligned consecutive lanes, which sum the squares among themselves.
    // The gate of chunk j is loaded one iteration ahead of its use.
    // With the down-projection the output rows are tokens: row t sums the R
    // output-tile rows t*R + r, which phase 2 already scaled by the weights.
    constexpr bool kDown = EPI == kEpiDown;
    const bool gated = EPI != kEpiPlain && has_y;
    const int RO = kDown ? 1 : R;                    // output rows per token in HBM
    const int RT = kDown ? 1 : RP;                   // output rows per token in the tile loops
    const size_t tokO = (size_t)H * RO * P;          // output row stride per token
    const IO* Zg = gated ? static_cast<const IO*>(a.gz) + ((size_t)b * T * H + hh) * RO * P : nullptr;
    IO* const Og = static_cast<IO*>(a.y) + ((size_t)b * T * H + hh) * RO * P;
    const bool padr = R != RP;  // padded ranks present (uniform)
    auto out_off = [&](int c0, int e) -> size_t {
      const int row = e / G16, gq = e % G16;
      if constexpr (kDown) return (size_t)(c0 + row) * tokO + gq * EG;
      return (size_t)(c0 + (row >> lgR)) * tokO + (padr ? rank_of(row) : (row & (RP - 1))) * P + gq * EG;
    };
    float gwr[EG];
    uint4 zr[KZ];
    if (gated) {
#pragma unroll
      for (int q = 0; q < EG; ++q) gwr[q] = a.gw[(size_t)hh * P + (ct % G16) * EG + q];
    }
    // down-projection weights of this lane's output-tile entries in phase 2:
    // rows rho = 16 rb + c all have rank c % R, columns 16 pb + 4 g .. + 3
    float dwr[kDown ? PBW : 1][4];
    if constexpr (kDown) {
#pragma unroll
      for (int u = 0; u < PBW; ++u) {
        const int pb = cw + kConsWaves * u;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          dwr[u][i4] = (pb < PB && (c & (RP - 1)) < R)
                           ? a.gdown[((size_t)hh * R + (c & (RP - 1))) * P + 16 * pb + 4 * g + i4]
                           : 0.f;
      }
    }
    auto load_z = [&](int jz) {
      const int ng = chunk_len(jz) * RT * G16;
#pragma unroll
      for (int k = 0; k < KZ; ++k) {
        const int e = ct + k * kCT;  // clamped duplicate past the tail, never used
        zr[k] = *reinterpret_cast<const uint4*>(Zg + out_off(jz * Q, e < ng ? e : ng - 1));
      }
    };
    auto store_y = [&](int jy) {
      const int c0 = jy * Q, ng = chunk_len(jy) * RP * G16;
      if (R == RP) {  // no padded ranks (uniform branch): every tile row is stored, no rank checks
        for (int e = ct; e < ng; e += kCT) {
          const int row = e / G16, gq = e % G16;
          *reinterpret_cast<uint4*>(Yg + (size_t)(c0 + (row >> lgR)) * tokX + (row & (RP - 1)) * P + gq * EG) =
              *reinterpret_cast<const uint4*>(sY + row * ldy + gq * EG);
        }
      } else {
        for (int e = ct; e < ng; e += kCT) {
          const int row = e / G16, gq = e % G16;
          if (real_row(row))
            *reinterpret_cast<uint4*>(Yg + gran_off(c0, e)) = *reinterpret_cast<const uint4*>(sY + row * ldy + gq * EG);
        }
      }
    };
    uint4 gres[KZ];
    auto gate_y = [&](int jy) {
      const int ng = chunk_len(jy) * RT * G16;
#pragma unroll
      for (int k = 0; k < KZ; ++k) {
        const int e = ct + k * kCT;
        if (e < ng) {  // whole rows: all G16 lanes of a row agree
          const int row = e / G16, gq = e % G16;
          float v[EG], z[EG];
          if constexpr (kDown) {
            Gran<IO>::unpack(*reinterpret_cast<const uint4*>(sY + row * RP * ldy + gq * EG), v);
#pragma unroll
            for (int r = 1; r < 8; ++r) {
              if (r < R) {
                float w[EG];
                Gran<IO>::unpack(*reinterpret_cast<const uint4*>(sY + (row * RP + r) * ldy + gq * EG), w);
#pragma unroll
                for (int q = 0; q < EG; ++q) v[q] += w[q];
              }
            }
          } else {
            Gran<IO>::unpack(*reinterpret_cast<const uint4*>(sY + row * ldy + gq * EG), v);
          }
          float ss = 0.f;
#pragma unroll
          for (int q = 0; q < EG; ++q) ss += v[q] * v[q];
          ss = lane_group_sum(ss, G16);
          const float inv = rsqrtf(ss * (1.0f / P) + a.geps);
          Gran<IO>::unpack(zr[k], z);
#pragma unroll
          for (int q = 0; q < EG; ++q) v[q] = gate_out(v[q], inv, gwr[q], z[q]);
          gres[k] = Gran<IO>::pack(v);
        }
      }
    };
    auto store_gated = [&](int jy) {
      const int c0 = jy * Q, ng = chunk_len(jy) * RT * G16;
#pragma unroll
      for (int k = 0; k < KZ; ++k) {
        const int e = ct + k * kCT;
        if (e < ng && (kDown || !padr || real_row(e / G16))) *reinterpret_cast<uint4*>(Og + out_off(c0, e)) = gres[k];
      }
    };
    for (int i = ck0; i <= ck1; ++i) {
      if (gated) {
        // results of chunk i-2, then the gate loads of chunk i-1, then the
        // stores: loads issued ahead of the stores never wait for them
        if (i >= ck0 + 2) gate_y(i - 2);
        if (i > ck0) load_z(i - 1);
        if (i >= ck0 + 2) store_gated(i - 2);
      } else if (has_y && i >= ck0 + 2) {
        store_y(i - 2);
      }
      // ---- phase 1: this wave's 16x16 blocks of S.M for chunk i-1 ----
      // Blocks (rb, kb), kb <= rb, are dealt round-robin to the 4 consumer
      // waves.  S^T = Bt Ct^T leaves the accumulator with 4 consecutive keys
      // per lane for one query, masked by the trapezoid decay and stored as
      // one 4-element run of row `query` of sSM (D x on the diagonal).
      if (i > ck0 && has_y) {
        const int j = i - 1;
        const PcBuf<IO, N, P> bf = getbuf(j);
        const PcCoef co = getcoef(j);
        const int rbn = (rows + 15) >> 4;
        const int nblk = rbn * (rbn + 1) / 2;
        // groups of up to kGrp blocks in straight-line code, so the LDS reads
        // of a group are all in flight before its first product
        constexpr int NBLK = RBM * (RBM + 1) / 2, NQ = (NBLK + kConsWaves - 1) / kConsWaves;
        constexpr int kGrp = NQ < 3 ? NQ : 3;
        for (int q0 = 0; q0 < NQ; q0 += kGrp) {
          int rbq[kGrp], kbq[kGrp];
          bool okq[kGrp];
#pragma unroll
          for (int q = 0; q < kGrp; ++q) {
            const int bi = cw + kConsWaves * (q0 + q);
            okq[q] = bi < nblk;
            int rem = okq[q] ? bi : 0, rb = 0;
            while (rem > rb) {  // block index -> (row block, key block), kb <= rb
              rem -= rb + 1;
              ++rb;
            }
            rbq[q] = rb;
            kbq[q] = rem;
          }
          Frag<IO> Bf[kGrp][NS], Cf[kGrp][NS];
          float4 kt[kGrp][4];
          float lq[kGrp], le[kGrp];
#pragma unroll
          for (int q = 0; q < kGrp; ++q) {
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {  // K = n in natural order (one 16-byte read each)
              Bf[q][ns].load8(bf.sB + (16 * kbq[q] + c) * LDN + 32 * ns + 8 * g);
              Cf[q][ns].load8(bf.sC + (16 * rbq[q] + c) * LDN + 32 * ns + 8 * g);
            }
            const int tq = (16 * rbq[q] + c) >> lgR;
            lq[q] = co.sTok[tq < Q ? tq : Q - 1].z;
            // first token after the key block (the factored mask's reference)
            const int tk1 = ((16 * kbq[q] + 15) >> lgR) + 1;
            le[q] = co.sTok[tk1 < Q ? tk1 : Q - 1].z;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int tk = (16 * kbq[q] + 4 * g + i4) >> lgR;
              kt[q][i4] = co.sTok[tk < Q ? tk : Q - 1];
            }
          }
#pragma unroll
          for (int q = 0; q < kGrp; ++q) {
            f32x4 St = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) mma(St, Bf[q][ns], Cf[q][ns]);
            const int rq = 16 * rbq[q] + c, tq = rq >> lgR;
            float v[4];
            if (kbq[q] < rbq[q]) {
              // below the diagonal every key precedes every query: one row
              // factor 2^{L_q - L_{e+1}} times the key factors
              const float rf = __builtin_amdgcn_exp2f(lq[q] - le[q]);
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) v[i4] = St[i4] * (rf * kt[q][i4].w);
            } else {
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const int rk = 16 * kbq[q] + 4 * g + i4, tk = rk >> lgR;
                float m = (tk <= tq) ? __builtin_amdgcn_exp2f(lq[q] - kt[q][i4].x) : 0.f;
                m += (tk < tq) ? __builtin_amdgcn_exp2f(lq[q] - kt[q][i4].y) : 0.f;
                v[i4] = St[i4] * m + ((rk == rq) ? Dh : 0.f);
              }
            }
            if (okq[q]) store4(sSM + rq * ldr + 16 * kbq[q] + 4 * g, v);
          }
        }
      }
      __syncthreads();
      // ---- phase 2: outputs and state update for this wave's p-blocks ----
      // Their work grows with the state size (the carried-state product and
      // the state update); from N = 128 on they are the longer side of the
      // second phase and run at raised priority.  Measured on the 1.5B-scale
      // shapes: N = 128 SISO 0.2826 -> 0.2770 ms with it; N = 64 MIMO R = 4,
      // whose producers' second phase is as long, 0.686 -> 0.696 ms with it.
      if constexpr (N >= 128) __builtin_amdgcn_s_setprio(2);
      if (i > ck0) {
        const int j = i - 1;
        const int c0 = j * Q, Lc = chunk_len(j);
        const PcBuf<IO, N, P> bf = getbuf(j);
        const PcCoef co = getcoef(j);
        const bool last_chunk = j == ck1 - 1;
#pragma unroll
        for (int u = 0; u < PBW; ++u) {
          const int pb = cw + kConsWaves * u;
          if (pb >= PB) continue;
          // X^T rows p, K = keys in natural order: the B operand of the
          // outputs' (S.M) product and of the state update
          Frag<IO> Xs[KSM];
#pragma unroll
          for (int ks = 0; ks < KSM; ++ks) Xs[ks].load8(bf.sXt + (16 * pb + c) * ldr + 32 * ks + 8 * g);
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
            // every row block's products first, then the y stores: a store to
            // the output tile between them would keep the next block's LDS
            // reads (which the compiler cannot tell apart from it) from being
            // issued ahead, and each product would wait a full LDS round trip
            f32x4 yacc[RBM];
            // C~ rows of the next row block are read while this block's
            // products run (two register sets)
            Frag<IO> Cf2[2][NS];
            auto load_cf = [&](int rb, Frag<IO> (&cf)[NS]) {
#pragma unroll
              for (int ns = 0; ns < NS; ++ns) {
                const IO* cr = bf.sC + (16 * rb + c) * LDN + 32 * ns + 4 * g;
                cf[ns].load44(cr, cr + 16);
              }
            };
            load_cf(0, Cf2[0]);
#pragma unroll
            for (int rb = 0; rb < RBM; ++rb) {
              const int rho = 16 * rb + c;
              f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
              // (LDS reads return in order: the row's decay first, so that
              // waiting for it does not wait for the tiles)
              const int tq = rho >> lgR;
              const float lqs = co.sTok[tq < Q ? tq : Q - 1].z;
              Frag<IO> SMf[KSM];
#pragma unroll
              for (int ks = 0; ks < KSM; ++ks)
                if (2 * ks <= rb) SMf[ks].load8(sSM + rho * ldr + 32 * ks + 8 * g);
              if (rb + 1 < RBM) load_cf(rb + 1, Cf2[(rb + 1) & 1]);
              // the reads above stay ahead of this block's products
              __builtin_amdgcn_sched_barrier(0);
              {
                Frag<IO>(&Cf)[NS] = Cf2[rb & 1];
#pragma unroll
                for (int ns = 0; ns < NS; ++ns) mma(acc, Hf[ns], Cf[ns]);
                acc = acc * __builtin_amdgcn_exp2f(lqs);
              }
#pragma unroll
              for (int ks = 0; ks < KSM; ++ks)
                if (2 * ks <= rb) mma(acc, Xs[ks], SMf[ks]);
              yacc[rb] = acc;
            }
#pragma unroll
            for (int rb = 0; rb < RBM; ++rb) {
              // y (row rho, columns 16pb + 4g .. +3) into the output tile
              // (down-projection: scaled by the weights of rank rho % R)
              const int rho = 16 * rb + c;
              float v[4] = {yacc[rb][0], yacc[rb][1], yacc[rb][2], yacc[rb][3]};
              if constexpr (kDown) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) v[i4] *= dwr[u][i4];
              }
              store4(sY + rho * ldy + 16 * pb + 4 * g, v);
            }
          }
          // state update and rotation into the next chunk's frame
          const float decE = expf(co.sMisc[0]);
          // all operands first (independent LDS reads), then the MFMA chains
          Frag<IO> Bs[NB][KSM];
          float2 r0[NB], r1[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks) Bs[nb][ks].load8(bf.sBt + (16 * nb + c) * ldr + 32 * ks + 8 * g);
            // this lane's pairs 8 nb + 2 g and 8 nb + 2 g + 1: one 16-byte read
            const float4 e = bf.sEnd[4 * nb + g];
            r0[nb] = make_float2(e.x, e.y);
            r1[nb] = make_float2(e.z, e.w);
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            f32x4 hacc = Hreg[u][nb] * decE;
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks) mma(hacc, Bs[nb][ks], Xs[ks]);
            float v[4] = {hacc[0], hacc[1], hacc[2], hacc[3]};
            rot2(v[0], v[1], r0[nb].x, r0[nb].y);
            rot2(v[2], v[3], r1[nb].x, r1[nb].y);
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
            const float tot = reduce_angle(sSeg[ct] + reinterpret_cast<const float*>(bf.sEnd + N / 4)[ct]);
            sSeg[ct] = tot;
            if (last_chunk) a.seg_angle[((size_t)seg * kp.batch * H + chain) * (N / 2) + ct] = tot;
          }
          if (ct == 0) {
            lsum += co.sMisc[0];
            if (last_chunk) a.seg_decay[(size_t)seg * kp.batch * H + chain] = lsum;
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
    }
    if (gated && ck1 > ck0) {
      gate_y(ck1 - 1);
      store_gated(ck1 - 1);
    } else if (has_y && ck1 > ck0) {
      store_y(ck1 - 1);
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

template <typename IO, int N, int P, int EPI, bool BCN, int LGR, bool SUMM = false>
hipError_t launch_pc_k(const PcParams& kp, size_t lds, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_pc_kernel<IO, N, P, EPI, BCN, LGR, SUMM>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((prefill_pc_kernel<IO, N, P, EPI, BCN, LGR, SUMM>), dim3(kp.nblocks), dim3(kPcThreads), lds, st,
                     kp);
  return hipGetLastError();
}

template <typename IO, int N, int P, int EPI, bool BCN>
hipError_t launch_pc_t(const Dims& d, const PrefillArgs& a, hipStream_t st, int mode, int nblocks) {
  // instances whose tiles fit at no height are never launched (the host
  // checks this first), so their kernels are not compiled
  if constexpr (PcLimits<IO, N, P>::kMaxRows == 0) {
    return hipErrorInvalidValue;
  } else {
    const size_t lds = PcLds<IO, N, P, BCN>::bytes(PcLimits<IO, N, P>::kMaxRows);
    if (lds > 160 * 1024) return hipErrorInvalidValue;  // (the host checks this first)
    PcParams kp;
    kp.a = a;
    kp.batch = d.batch;
    kp.heads = d.heads;
    kp.R = d.R;
    kp.lgR = pad_rank_log2(d.R);
    kp.Q = d.Q;
    kp.mode = mode;
    kp.nblocks = nblocks;
    // Instances with the rank (and, but for the gated per-rank epilogue, the
    // tile height) fixed at compile time, where they measured faster than the
    // one that takes both from kp (A/B on one box; the second figure adds the
    // fixed tile height): bf16 ranks 3-4 (MIMO R = 4 prefill 0.689 -> 0.594
    // -> 0.573 ms, with the BC normalisation 0.861 -> 0.739 -> 0.621 ms,
    // down-projected and gated 0.850 -> 0.700 -> 0.665 ms, gated 0.830 ->
    // 0.713 ms but 0.739 ms with the fixed height); bf16 rank 1 in the segment passes
    // (16K-token SISO path 0.2745 -> 0.267 ms) and with the BC normalisation
    // (0.336 -> 0.318 -> 0.301 ms); fp32 rank 1 (0.881 -> 0.828 -> 0.810 ms).
    // The fused bf16 rank-1 pass without the BC normalisation keeps the
    // general instance: 0.2787 -> 0.284 ms plain, 0.313 -> 0.317 gated, and
    // 0.280 -> 0.286 ms with only the tile height fixed.
    const bool full = EPI == kEpiGate || kp.Q == (PcLimits<IO, N, P>::kMaxRows >> kp.lgR);
    // segment summaries (always the plain output) in instances of their own
    if constexpr (EPI == kEpiPlain) {
      if (mode == kPcSummary && full && kp.lgR == 0) return launch_pc_k<IO, N, P, EPI, BCN, 0, true>(kp, lds, st);
      if constexpr (sizeof(IO) == 2) {
        if (mode == kPcSummary && full && kp.lgR == 2) return launch_pc_k<IO, N, P, EPI, BCN, 2, true>(kp, lds, st);
      }
    }
    if constexpr (sizeof(IO) == 2) {
      if (full && kp.lgR == 0 && (mode != kPcFused || BCN)) return launch_pc_k<IO, N, P, EPI, BCN, 0>(kp, lds, st);
      if (full && kp.lgR == 2) return launch_pc_k<IO, N, P, EPI, BCN, 2>(kp, lds, st);
    } else {
      if (full && kp.lgR == 0) return launch_pc_k<IO, N, P, EPI, BCN, 0>(kp, lds, st);
    }
    return launch_pc_k<IO, N, P, EPI, BCN, -1>(kp, lds, st);
  }
}

template <typename IO, int N, int EPI, bool BCN>
hipError_t pc_p(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nb) {
  switch (d.P) {
    case 16: return launch_pc_t<IO, N, 16, EPI, BCN>(d, a, s, mode, nb);
    case 32: return launch_pc_t<IO, N, 32, EPI, BCN>(d, a, s, mode, nb);
    case 64: return launch_pc_t<IO, N, 64, EPI, BCN>(d, a, s, mode, nb);
    default: return launch_pc_t<IO, N, 128, EPI, BCN>(d, a, s, mode, nb);
  }
}

template <typename IO, int EPI, bool BCN>
hipError_t pc_n(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nb) {
  switch (d.N) {
    case 16: return pc_p<IO, 16, EPI, BCN>(d, a, s, mode, nb);
    case 32: return pc_p<IO, 32, EPI, BCN>(d, a, s, mode, nb);
    case 64: return pc_p<IO, 64, EPI, BCN>(d, a, s, mode, nb);
    case 128: return pc_p<IO, 128, EPI, BCN>(d, a, s, mode, nb);
    default: return pc_p<IO, 256, EPI, BCN>(d, a, s, mode, nb);
  }
}

template <int EPI, bool BCN>
hipError_t launch_pc(const Dims& d, const PrefillArgs& a, hipStream_t s, int mode, int nblocks) {
  return d.bf16 ? pc_n<bf16, EPI, BCN>(d, a, s, mode, nblocks) : pc_n<float, EPI, BCN>(d, a, s, mode, nblocks);
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
    M3_CASE(256, 16) M3_CASE(256, 32) M3_CASE(256, 64) M3_CASE(256, 128)
#undef M3_CASE
    default: return 0;
  }
}

// Whether the BC-normalisation instance of <IO, N, P> fits the LDS (its
// weights and partial sums come on top of the plain instance's tiles).
template <typename IO>
bool pc_bcn_fits(const Dims& d) {
  switch (d.N * 1000 + d.P) {
#define M3_CASE(NN, PP) \
  case NN * 1000 + PP: return PcLds<IO, NN, PP, true>::bytes(PcLimits<IO, NN, PP>::kMaxRows) <= 160 * 1024;
    M3_CASE(16, 16) M3_CASE(16, 32) M3_CASE(16, 64) M3_CASE(16, 128)
    M3_CASE(32, 16) M3_CASE(32, 32) M3_CASE(32, 64) M3_CASE(32, 128)
    M3_CASE(64, 16) M3_CASE(64, 32) M3_CASE(64, 64) M3_CASE(64, 128)
    M3_CASE(128, 16) M3_CASE(128, 32) M3_CASE(128, 64) M3_CASE(128, 128)
    M3_CASE(256, 16) M3_CASE(256, 32) M3_CASE(256, 64) M3_CASE(256, 128)
#undef M3_CASE
    default: return false;
  }
}

}  // namespace
}  // namespace m3
