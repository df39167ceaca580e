/*
 * mamba3.h -- C ABI of the MI355X (gfx950) Mamba-3 SSM scan library.
 *
 * The library evaluates the Mamba-3 state-space recurrence: exponential-
 * trapezoid (second-order) discretisation with a data-dependent rotating
 * ("complex", RoPE-trick) state, in SISO (rank 1) and MIMO (rank R) form,
 * as a chunked parallel prefill over a prompt and as a single-token decode
 * step.  Sources (web pages on Mamba-3, which print no equations):
 *   lilting.ch, "Together AIがMamba-3を発表、長文推論でTransformer比約7倍の速度と
 *   複素数値SSM", section "アーキテクチャ改善":
 *     "1. 指数台形離散化"  -- second-order rule mixing current and previous input;
 *     "2. 複素数値状態"    -- N real state dims = N/2 complex pairs, realised as
 *                            block-diagonal 2x2 rotations of real vectors;
 *     "3. MIMO SSM"        -- rank-r input/output coupling (r = 4 on the page);
 *   same article, section "カーネル実装の多層構成": a prefill kernel and a
 *   separate latency-oriented decode kernel.
 *
 * Definition computed (per batch row b and head h, for each token t):
 *     alpha = exp(dt_t * A_h),  beta = (1 - lam_t) dt_t,  gamma = lam_t dt_t
 *     G     = alpha h + beta sum_r x_prev[r] (x) B_prev[r]          (P x N)
 *     h     = RotPairs(G, theta_t) + gamma sum_r x_t[r] (x) B_t[r]
 *     y_t[r]= h C_t[r] + D_h x_t[r]
 *     (B_prev, x_prev) = (B_t, x_t)
 * RotPairs rotates state columns (2j, 2j+1) by theta_t[j]:
 *     (a, b) -> (a cos - b sin, a sin + b cos).
 * theta is the per-token angle (already scaled by dt), shared by the P rows
 * and the R ranks; dt, lam, theta, A and D are shared by the R ranks.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP device memory of the
 *     current device); every call is asynchronous on `stream` (a hipStream_t
 *     passed as void*; NULL = the default stream).  Nothing synchronises.
 *   - The caller owns every buffer.  The library allocates no device memory;
 *     the only device memory of its own is the 16 MiB scratch array of
 *     mamba3_prefill_noalloc, part of its loaded code object on each GPU.
 *   - Tensors are dense, row-major, in the layouts given below, with base
 *     pointers aligned to 16 bytes.
 *   - I/O dtype (x, B, C, y, B_prev, x_prev) is fp32 or bf16 as dims.io_dtype
 *     says; dt, lam, theta, A, D and the state h are always fp32.
 *   - Errors detectable on the host (NULL pointer, bad shape, unsupported
 *     size, misalignment, short workspace) return a negative m3_status BEFORE
 *     any HIP call; m3_last_error() then describes the problem.  A failed
 *     launch returns M3_ERR_HIP.  Faults inside a kernel surface at the
 *     caller's next synchronisation.  No NaN/Inf checks are made.
 */
#ifndef MAMBA3_H
#define MAMBA3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define M3_ABI_VERSION 6

typedef enum {
  M3_OK = 0,
  M3_ERR_NULL = -1,        /* a required pointer is NULL                         */
  M3_ERR_SHAPE = -2,       /* a size is negative or zero where it must be > 0    */
  M3_ERR_DTYPE = -3,       /* io_dtype is not one of m3_dtype                    */
  M3_ERR_ALIGN = -4,       /* a tensor base pointer is not 16-byte aligned       */
  M3_ERR_UNSUPPORTED = -5, /* sizes valid but outside the compiled set (below)   */
  M3_ERR_WORKSPACE = -6,   /* workspace smaller than the required size           */
  M3_ERR_HIP = -7          /* a HIP launch or runtime call failed                */
} m3_status;

typedef enum { M3_F32 = 0, M3_BF16 = 1 } m3_dtype;

/* Discretisation rule: the per-token weights (alpha, beta, gamma) in
 *     h = Rot(theta)(alpha h + beta sum_r x_prev[r] (x) B_prev[r]) + gamma sum_r x[r] (x) B[r]
 * lilting.ch Mamba-3 article, "1. 指数台形離散化" (its table of methods) and
 * the table "Mamba-2とMamba-3の比較".  alpha = exp(dt A) for every rule.
 *   M3_DISC_EXP_TRAPEZOID      Mamba-3 (default): beta = (1-lam) dt, gamma = lam dt
 *   M3_DISC_DECAYED_TRAPEZOID  textbook trapezoid, the previous input decays
 *                              with the state: beta = alpha (1-lam) dt, gamma = lam dt
 *   M3_DISC_EXP_EULER          Mamba-2, first order: beta = 0, gamma = dt (lam unused) */
typedef enum {
  M3_DISC_EXP_TRAPEZOID = 0,
  M3_DISC_DECAYED_TRAPEZOID = 1,
  M3_DISC_EXP_EULER = 2
} m3_disc;

/* Problem sizes.  Supported set:
 *   batch >= 1, heads >= 1 (batch*heads <= 2^21),
 *   headdim P in {16, 32, 64, 128},
 *   dstate  N in {16, 32, 64, 128, 256}  (N/2 complex pairs),
 *   rank    R in 1..8                    (1 = SISO, > 1 = MIMO; the prefill
 *                                         tiles hold R rounded up to a power
 *                                         of two rows per token, the padded
 *                                         rows with x = 0),
 *   chunk   Q in {16, 32, 64}            (prefill block length; the result
 *                                         does not depend on it: the library
 *                                         tiles with the largest height <= Q
 *                                         whose tiles fit, halving down to 16
 *                                         tokens, or 4 for R >= 3),
 *   io_dtype in m3_dtype,
 *   disc in m3_disc (0, the default, when the struct is zero-initialised).
 * Support does not depend on the chunk: a size accepted at chunk 16 is
 * accepted at 32 and 64.  Within that set M3_ERR_UNSUPPORTED is returned for
 *   - prefill with fp32 I/O and N = 256, except P = 16 with R <= 2: the
 *     producer/consumer kernel holds a chunk's B and C rows in producer
 *     registers (16 KiB at most; a 32-row tile of 256 fp32 values per row is
 *     32 KiB), and the single-role kernel's LDS (B~, C~ at a 264-float pitch,
 *     B~^T, X^T and a copy of the state: 2 x 33.8 + 36.9 + 2.3 + 16.9 KiB plus
 *     the angles at 32 rows) fits 160 KiB only for P = 16;
 *   - prefill with fp32 I/O, P = 128, N = 128 and R >= 3: two 32-row tile
 *     buffers (B~, C~ at a 132-float pitch, B~^T, X^T: 70 KiB each) and the
 *     score and output tiles need 165 KiB of LDS, and the single-role kernel
 *     fits this size only for R <= 2;
 *   - decode with P = 128, N = 256 and R >= 5: the matrix-core kernel's
 *     state staging rows (128 x 260 x 4 B = 130 KiB) and rank operands exceed
 *     160 KiB of LDS, and the VALU kernel serves R <= 4.
 * Values <= 0 return M3_ERR_SHAPE.  The backward pass has its own, smaller
 * set (mamba3_prefill_backward). */
typedef struct {
  int32_t batch, heads, headdim, dstate, rank, chunk;
  int32_t io_dtype;
  int32_t disc;
} m3_dims;

/* Recurrent state of every (batch, head): the fixed-size memory an SSM
 * carries from token to token instead of a Transformer's growing key/value
 * cache (lilting.ch Mamba-3 article, section "SSMとは何か、Transformerの推論
 * コスト問題"; the prefill hands it to the decode steps).  It is kept in the
 * LAB frame (the frame of the definition above; no accumulated rotation is
 * folded in):
 *   h       fp32      (batch, heads, P, N)
 *   B_prev  io dtype  (batch, heads, R, N)   last token's B  (pending input)
 *   x_prev  io dtype  (batch, heads, R, P)   last token's x
 * A fresh sequence is all zeros (m3_state_zero). */
typedef struct {
  float* h;
  void* B_prev;
  void* x_prev;
} m3_state;

/* ABI version (M3_ABI_VERSION). */
int m3_abi_version(void);

/* Thread-local, NUL-terminated description of the last non-OK status returned
 * on this thread (empty string if none).  Owned by the library. */
const char* m3_last_error(void);

/* Host only.  Byte sizes of the three state buffers for `dims`.  Any output
 * pointer may be NULL. */
int m3_state_bytes(const m3_dims* dims, size_t* h_bytes, size_t* bprev_bytes,
                   size_t* xprev_bytes);

/* Zero the whole state (h, B_prev, x_prev): the start of a fresh sequence
 * (the state of the section cited at m3_state, before any token).  Uses a
 * fill kernel (no memset node), so it may be captured in a HIP graph. */
int m3_state_zero(const m3_dims* dims, m3_state* state, void* stream);

/* Copy a state from caller buffers (same layouts as m3_state) into `dst`:
 * resuming a sequence from its fixed-size state (section cited at m3_state).
 * Source and destination must not overlap. */
int m3_state_load(const m3_dims* dims, m3_state* dst, const float* h,
                  const void* B_prev, const void* x_prev, void* stream);

/* Copy `src` out into caller buffers (same layouts): the whole memory of a
 * sequence after its last token (section cited at m3_state).  Must not
 * overlap. */
int m3_state_readout(const m3_dims* dims, const m3_state* src, float* h,
                     void* B_prev, void* x_prev, void* stream);

/* Host only.  Workspace bytes that mamba3_prefill needs for (dims, seqlen).
 * 0 when the prompt is processed by one fused pass; >0 when the library
 * splits long prompts of few (batch, head) chains into segments whose start
 * states are found by a scan over segment summaries. */
int mamba3_prefill_workspace_bytes(const m3_dims* dims, int32_t seqlen, size_t* bytes);

/* Chunked parallel prefill of `seqlen` tokens for every (batch, head).
 *   x      io    (batch, seqlen, heads, R, P)
 *   B, C   io    (batch, seqlen, heads, R, N)
 *   dt     fp32  (batch, seqlen, heads)
 *   lam    fp32  (batch, seqlen, heads)
 *   theta  fp32  (batch, seqlen, heads, N/2)   per-token angles (scaled by dt)
 *   A, D   fp32  (heads)
 *   state  in: the state before the prompt; out: the state after it (in place)
 *   y      io    (batch, seqlen, heads, R, P)   output; must not alias inputs
 *   workspace / workspace_bytes: device scratch of at least
 *     mamba3_prefill_workspace_bytes(dims, seqlen) bytes (may be NULL if 0).
 * seqlen == 0 is a no-op that returns M3_OK.  Results match the sequential
 * definition up to rounding: fp32 state and accumulation; with bf16 I/O the
 * rotated B/C, the masked score tile and the carried state are rounded to
 * bf16 as matrix-core operands.
 * Domain: any finite inputs with dt * A <= 0 (decay).  A token's log-decay
 * dt * A below -32 (a state reset) is raised to -32 inside the chunked
 * kernels: such a token passes e^-32 ~ 1.3e-14 of the state before it
 * instead of less, a change far below fp32 resolution, and no intermediate
 * overflows for any finite decay.  Angles of any size are accepted (the bf16
 * path reduces them to one revolution before the hardware sine). */
int mamba3_prefill(const m3_dims* dims, int32_t seqlen, const void* x, const void* B,
                   const void* C, const float* dt, const float* lam, const float* theta,
                   const float* A, const float* D, m3_state* state, void* y,
                   void* workspace, size_t workspace_bytes, void* stream);

/* mamba3_prefill for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace.  Where mamba3_prefill needs a
 * segment workspace (long prompts of few chains), this call uses the
 * library's own device scratch instead: a file-scope device array of 16 MiB
 * per GPU, held until the process ends.  Sizes whose workspace
 * (mamba3_prefill_workspace_bytes) exceeds 16 MiB return M3_ERR_UNSUPPORTED
 * before any HIP call.  The call allocates nothing.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  The scratch
 * needs no clearing between calls (a call writes everything it reads), and
 * results are identical to mamba3_prefill's.  The scratch is the current
 * device's, so `stream` must belong to the current device.  ABI version 6. */
int mamba3_prefill_noalloc(const m3_dims* dims, int32_t seqlen, const void* x, const void* B,
                           const void* C, const float* dt, const float* lam, const float* theta,
                           const float* A, const float* D, m3_state* state, void* y, void* stream);

/* One recurrent step: one new token for every (batch, head).
 *   x      io    (batch, heads, R, P)
 *   B, C   io    (batch, heads, R, N)
 *   dt, lam fp32 (batch, heads);  theta fp32 (batch, heads, N/2)
 *   A, D   fp32  (heads)
 *   state  updated in place (h streamed once: read once, written once)
 *   y      io    (batch, heads, R, P); must not alias inputs or state.
 * dims.chunk is ignored. */
int mamba3_decode_step(const m3_dims* dims, const void* x, const void* B, const void* C,
                       const float* dt, const float* lam, const float* theta,
                       const float* A, const float* D, m3_state* state, void* y,
                       void* stream);

/* Output epilogue: pre-gate grouped RMSNorm, fused into the store of y
 * (ai-flow-lab.com Mamba-3 summary, section "実装とカーネル最適化": a grouped
 * RMSNorm before the output gate).  Each (token, head, rank) row of P output
 * channels s[0..P) of the scan is one group:
 *   y[p] = weight[head][p] * s[p] / sqrt(mean_p s[p]^2 + eps) * silu(z[p]),
 *   silu(v) = v / (1 + exp(-v)).
 * With down != NULL the R rank rows of a (token, head) are first folded into
 * one row of P channels (lilting.ch Mamba-3 article, "3. MIMO SSM": the
 * rank-r output returns to the channels), s[p] = sum_r down[head][r][p] *
 * scan[r][p], and that row is the group; y and z then have no rank axis.
 *   z       io    same layout as y (the gate input)
 *   weight  fp32  (heads, P)
 *   eps     >= 0
 *   down    fp32  (heads, R, P), or NULL: no down-projection
 * All pointers are device pointers, 16-byte aligned, owned by the caller. */
typedef struct {
  const void* z;
  const float* weight;
  float eps;
  const float* down;
} m3_gate;

/* mamba3_prefill with the epilogue: y receives the gated, normalised output
 * (the raw scan output is not written); with gate->down, y and gate->z are
 * (batch, seqlen, heads, P).  Same arguments and errors as
 * mamba3_prefill, plus M3_ERR_NULL / M3_ERR_ALIGN for gate, gate->z,
 * gate->weight, M3_ERR_SHAPE for a negative or NaN eps, and
 * M3_ERR_UNSUPPORTED for shapes that only the single-role prefill kernel
 * handles (fp32 I/O with tiles too large for the producer/consumer kernel). */
int mamba3_prefill_gated(const m3_dims* dims, int32_t seqlen, const void* x, const void* B,
                         const void* C, const float* dt, const float* lam, const float* theta,
                         const float* A, const float* D, const m3_gate* gate, m3_state* state,
                         void* y, void* workspace, size_t workspace_bytes, void* stream);

/* mamba3_decode_step with the epilogue (z and y of shape (batch, heads, R, P),
 * or (batch, heads, P) with gate->down). */
int mamba3_decode_step_gated(const m3_dims* dims, const void* x, const void* B, const void* C,
                             const float* dt, const float* lam, const float* theta,
                             const float* A, const float* D, const m3_gate* gate, m3_state* state,
                             void* y, void* stream);

/* BC normalisation (ai-flow-lab.com Mamba-3 summary, section
 * "実装とカーネル最適化": BC/QK normalisation, the QKNorm of attention applied
 * to the SSM's B and C; lilting.ch Mamba-3 article, comparison table,
 * normalisation row).  Before the scan uses them (and before any rotation),
 * every (token, head, rank) row of N channels of B and of C is normalised by
 * its RMS and scaled per channel:
 *   B'[n] = b_weight[head][n] * B[n] / sqrt(mean_n B[n]^2 + eps),
 *   C'[n] = c_weight[head][n] * C[n] / sqrt(mean_n C[n]^2 + eps).
 * The pending B_prev in the state stays the raw B of the last token and is
 * normalised the same way where the recurrence uses it.
 *   b_weight, c_weight  fp32 (heads, N), device pointers, 16-byte aligned
 *   eps                 >= 0 */
typedef struct {
  const float* b_weight;
  const float* c_weight;
  float eps;
} m3_bcnorm;

/* mamba3_prefill with optional BC normalisation (bcnorm, NULL: none) and an
 * optional output epilogue (gate, NULL: the raw scan output, as
 * mamba3_prefill; otherwise as mamba3_prefill_gated).  Same errors as those
 * two, plus M3_ERR_NULL / M3_ERR_ALIGN for bcnorm's weights, M3_ERR_SHAPE for
 * a negative or NaN bcnorm->eps, and M3_ERR_UNSUPPORTED for sizes whose
 * normalising prefill tiles do not fit (fp32 shapes served only by the
 * single-role kernel; bf16 with N = 64 and P = 16). */
int mamba3_prefill_ex(const m3_dims* dims, int32_t seqlen, const void* x, const void* B, const void* C,
                      const float* dt, const float* lam, const float* theta, const float* A, const float* D,
                      const m3_bcnorm* bcnorm, const m3_gate* gate, m3_state* state, void* y, void* workspace,
                      size_t workspace_bytes, void* stream);

/* mamba3_decode_step with optional BC normalisation and output epilogue. */
int mamba3_decode_step_ex(const m3_dims* dims, const void* x, const void* B, const void* C, const float* dt,
                          const float* lam, const float* theta, const float* A, const float* D,
                          const m3_bcnorm* bcnorm, const m3_gate* gate, m3_state* state, void* y, void* stream);

/* Backward pass of mamba3_prefill (training): the gradients of
 *   L = sum_t <dy_t, y_t> + <dh_final, h_T>
 * with respect to every input of a prefill that started from `state0`
 * (lilting.ch Mamba-3 article, "アーキテクチャ改善" 1-3; the exact derivative
 * of the recurrence that mamba3_prefill computes, under dims->disc).  All
 * gradients are fp32 device arrays in the layouts of the quantities they
 * belong to; dA and dD are summed over the batch.  The pending pair of the
 * final state is a copy of the last token's (B, x): a caller with cotangents
 * for it adds them to dB and dx of that token. */
typedef struct {
  float* dx;       /* (batch, seqlen, heads, R, P) */
  float* dB;       /* (batch, seqlen, heads, R, N) */
  float* dC;       /* (batch, seqlen, heads, R, N) */
  float* ddt;      /* (batch, seqlen, heads) */
  float* dlam;     /* (batch, seqlen, heads) */
  float* dtheta;   /* (batch, seqlen, heads, N/2) */
  float* dA;       /* (heads) */
  float* dD;       /* (heads) */
  float* dh0;      /* (batch, heads, P, N): of state0.h */
  float* dB_prev;  /* (batch, heads, R, N): of state0.B_prev */
  float* dx_prev;  /* (batch, heads, R, P): of state0.x_prev */
} m3_grads;

/* Workspace of mamba3_prefill_backward: with units of 64 / R tokens and
 * U = ceil(seqlen R / 64) units per chain, two P x N fp32 slots per unit (the
 * state's entry value and the adjoint after the unit) and one per chain (the
 * adjoint of the entry value), batch * heads * (2 U + 1) * P * N * 4 bytes,
 * then per-unit scalars: each of e^{lE} (U), the end angle's (cos, sin)
 * (U N), the first-token terms (2 U), the unit sums (2 U) and the chain sums
 * (2), times batch * heads * 4 bytes, rounded up to 256 bytes. */
int mamba3_prefill_backward_workspace_bytes(const m3_dims* dims, int32_t seqlen, size_t* bytes);

/* x, B, C, dt, lam, theta, A, D as given to mamba3_prefill; state0 the state
 * the prefill started from (read only); dy (io dtype, y's layout) the
 * cotangent of y; dh_final (fp32 (batch, heads, P, N)) that of the final h,
 * or NULL for zero.  dims->chunk is ignored.  Errors as mamba3_prefill, plus
 * M3_ERR_NULL / M3_ERR_ALIGN for grads and its arrays, M3_ERR_UNSUPPORTED
 * unless R is 1, 2 or 4 and P, N are multiples of 16 with P, N <= 128 and
 * P * N <= 8192, and M3_ERR_WORKSPACE for a short workspace. */
int mamba3_prefill_backward(const m3_dims* dims, int32_t seqlen, const void* x, const void* B, const void* C,
                            const float* dt, const float* lam, const float* theta, const float* A,
                            const float* D, const m3_state* state0, const void* dy, const float* dh_final,
                            const m3_grads* grads, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA3_H */
