// C ABI of the Mamba-3 scan library: argument validation and dispatch.
//
// Every host-detectable problem is reported with a negative m3_status before
// any HIP call is made, so the whole validation layer runs (and is tested)
// on machines without a GPU.  See include/mamba3.h for the contract.
#include "../../include/mamba3.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "m3_kernels.hpp"

namespace {

thread_local char g_err[512] = {0};

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = 0;
  return M3_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t io_size(const m3_dims* d) { return d->io_dtype == M3_BF16 ? 2 : 4; }

// Shape / dtype / support checks shared by every entry point.  `need_chunk`
// is false for the decode step (which ignores dims.chunk).
int check_dims(const m3_dims* d, bool need_chunk, m3::Dims* out) {
  if (!d) return fail(M3_ERR_NULL, "dims is NULL");
  if (d->batch <= 0 || d->heads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->rank <= 0)
    return fail(M3_ERR_SHAPE, "batch, heads, headdim, dstate and rank must be > 0 (got %d %d %d %d %d)",
                d->batch, d->heads, d->headdim, d->dstate, d->rank);
  if (need_chunk && d->chunk <= 0) return fail(M3_ERR_SHAPE, "chunk must be > 0 (got %d)", d->chunk);
  if (d->io_dtype != M3_F32 && d->io_dtype != M3_BF16)
    return fail(M3_ERR_DTYPE, "io_dtype %d is neither M3_F32 nor M3_BF16", d->io_dtype);
  if ((int64_t)d->batch * d->heads > (int64_t)(1 << 21))
    return fail(M3_ERR_UNSUPPORTED, "batch*heads = %lld exceeds 2^21",
                (long long)((int64_t)d->batch * d->heads));
  if (d->dstate % 2) return fail(M3_ERR_UNSUPPORTED, "dstate %d is odd (N/2 complex pairs)", d->dstate);
  if (d->disc < M3_DISC_EXP_TRAPEZOID || d->disc > M3_DISC_EXP_EULER)
    return fail(M3_ERR_UNSUPPORTED, "disc %d is not one of m3_disc", d->disc);
  m3::Dims m;
  m.batch = d->batch;
  m.heads = d->heads;
  m.P = d->headdim;
  m.N = d->dstate;
  m.R = d->rank;
  m.Q = need_chunk ? d->chunk : 64;
  m.bf16 = d->io_dtype == M3_BF16;
  m.disc = d->disc;
  const bool supported = need_chunk ? m3::prefill_supported(m) : m3::decode_supported(m);
  if (!supported)
    return fail(M3_ERR_UNSUPPORTED,
                "unsupported sizes headdim=%d dstate=%d rank=%d chunk=%d %s (supported: headdim in "
                "{16,32,64,128}, dstate in {16,32,64,128,256}, rank 1..8, chunk in {16,32,64}, and tiles "
                "that fit the LDS at some tile height; mamba3.h lists the exclusions)",
                d->headdim, d->dstate, d->rank, d->chunk, d->io_dtype == M3_BF16 ? "bf16" : "f32");
  *out = m;
  return M3_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(M3_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(M3_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return M3_OK;
}

int check_state(const m3_state* s, const char* what) {
  if (!s) return fail(M3_ERR_NULL, "%s is NULL", what);
  int st;
  if ((st = check_ptr(s->h, "state.h")) != M3_OK) return st;
  if ((st = check_ptr(s->B_prev, "state.B_prev")) != M3_OK) return st;
  if ((st = check_ptr(s->x_prev, "state.x_prev")) != M3_OK) return st;
  return M3_OK;
}

void state_sizes(const m3_dims* d, size_t* hb, size_t* bb, size_t* xb) {
  const size_t chains = (size_t)d->batch * d->heads;
  *hb = chains * d->headdim * d->dstate * sizeof(float);
  *bb = chains * d->rank * d->dstate * io_size(d);
  *xb = chains * d->rank * d->headdim * io_size(d);
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(M3_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Segment plan for the prefill.  Chains (batch*heads) that already fill the
// chip run one fused pass.  Few long chains are split into nseg segments so
// that about 256 workgroups (one per MI355X compute unit) run at once; each
// segment keeps at least 4 chunks.  Deterministic in (dims, seqlen) only.
constexpr int kTargetWorkgroups = 256;
constexpr int kMinSegChunks = 4;
constexpr int kMaxSegments = 64;

void plan_segments(const m3::Dims& m, int seqlen, int* nseg, int* seg_chunks) {
  const int nchunks = (seqlen + m.Q - 1) / m.Q;
  const int chains = m.batch * m.heads;
  int g = 1;
  if (chains < kTargetWorkgroups / 2) {
    g = (kTargetWorkgroups + chains - 1) / chains;
    if (g > kMaxSegments) g = kMaxSegments;
    const int gmax = nchunks / kMinSegChunks;
    if (g > gmax) g = gmax;
    if (g < 1) g = 1;
  }
  if (g == 1) {
    *nseg = 1;
    *seg_chunks = nchunks;
    return;
  }
  const int sc = (nchunks + g - 1) / g;
  *seg_chunks = sc;
  *nseg = (nchunks + sc - 1) / sc;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace layout for the segment path: seg_state | seg_decay | seg_angle.
size_t workspace_for(const m3::Dims& m, int nseg) {
  if (nseg <= 1) return 0;
  const size_t cs = (size_t)nseg * m.batch * m.heads;
  return align256(cs * m.P * m.N * sizeof(float)) + align256(cs * sizeof(float)) +
         align256(cs * (m.N / 2) * sizeof(float));
}

}  // namespace

extern "C" {

int m3_abi_version(void) { return M3_ABI_VERSION; }

const char* m3_last_error(void) { return g_err; }

int m3_state_bytes(const m3_dims* dims, size_t* h_bytes, size_t* bprev_bytes, size_t* xprev_bytes) {
  m3::Dims m;
  int st = check_dims(dims, false, &m);
  if (st != M3_OK) return st;
  size_t hb, bb, xb;
  state_sizes(dims, &hb, &bb, &xb);
  if (h_bytes) *h_bytes = hb;
  if (bprev_bytes) *bprev_bytes = bb;
  if (xprev_bytes) *xprev_bytes = xb;
  return ok();
}

int m3_state_zero(const m3_dims* dims, m3_state* state, void* stream) {
  m3::Dims m;
  int st = check_dims(dims, false, &m);
  if (st != M3_OK) return st;
  if ((st = check_state(state, "state")) != M3_OK) return st;
  size_t hb, bb, xb;
  state_sizes(dims, &hb, &bb, &xb);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* const p[3] = {state->h, state->B_prev, state->x_prev};
  const size_t n[3] = {hb, bb, xb};
  const hipError_t e = m3::launch_fill_zero3(p, n, s);
  return hip_status(e, "m3_state_zero");
}

int m3_state_load(const m3_dims* dims, m3_state* dst, const float* h, const void* B_prev,
                  const void* x_prev, void* stream) {
  m3::Dims m;
  int st = check_dims(dims, false, &m);
  if (st != M3_OK) return st;
  if ((st = check_state(dst, "dst")) != M3_OK) return st;
  if ((st = check_ptr(h, "h")) != M3_OK) return st;
  if ((st = check_ptr(B_prev, "B_prev")) != M3_OK) return st;
  if ((st = check_ptr(x_prev, "x_prev")) != M3_OK) return st;
  size_t hb, bb, xb;
  state_sizes(dims, &hb, &bb, &xb);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* const d[3] = {dst->h, dst->B_prev, dst->x_prev};
  const void* const from[3] = {h, B_prev, x_prev};
  const size_t n[3] = {hb, bb, xb};
  const hipError_t e = m3::launch_copy3(d, from, n, s);
  return hip_status(e, "m3_state_load");
}

int m3_state_readout(const m3_dims* dims, const m3_state* src, float* h, void* B_prev, void* x_prev,
                     void* stream) {
  m3::Dims m;
  int st = check_dims(dims, false, &m);
  if (st != M3_OK) return st;
  if ((st = check_state(src, "src")) != M3_OK) return st;
  if ((st = check_ptr(h, "h")) != M3_OK) return st;
  if ((st = check_ptr(B_prev, "B_prev")) != M3_OK) return st;
  if ((st = check_ptr(x_prev, "x_prev")) != M3_OK) return st;
  size_t hb, bb, xb;
  state_sizes(dims, &hb, &bb, &xb);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* const d[3] = {h, B_prev, x_prev};
  const void* const from[3] = {src->h, src->B_prev, src->x_prev};
  const size_t n[3] = {hb, bb, xb};
  const hipError_t e = m3::launch_copy3(d, from, n, s);
  return hip_status(e, "m3_state_readout");
}

int mamba3_prefill_workspace_bytes(const m3_dims* dims, int32_t seqlen, size_t* bytes) {
  m3::Dims m;
  int st = check_dims(dims, true, &m);
  if (st != M3_OK) return st;
  if (!bytes) return fail(M3_ERR_NULL, "bytes is NULL");
  if (seqlen < 0) return fail(M3_ERR_SHAPE, "seqlen %d < 0", seqlen);
  m.Q = m3::prefill_tile_chunk(m);
  int nseg = 1, sc = 0;
  if (seqlen > 0) plan_segments(m, seqlen, &nseg, &sc);
  *bytes = workspace_for(m, nseg);
  return ok();
}

}  // extern "C"

namespace {

// Gate argument checks; *gz stays nullptr without a gate.
int check_gate(const m3_gate* gate, const void** gz, const float** gw, float* geps, const float** gdown) {
  *gz = nullptr;
  *gw = nullptr;
  *geps = 0.f;
  *gdown = nullptr;
  if (!gate) return fail(M3_ERR_NULL, "gate is NULL");
  int st;
  if ((st = check_ptr(gate->z, "gate.z")) != M3_OK) return st;
  if ((st = check_ptr(gate->weight, "gate.weight")) != M3_OK) return st;
  if (!(gate->eps >= 0.f)) return fail(M3_ERR_SHAPE, "gate.eps must be >= 0 (got %g)", (double)gate->eps);
  if (gate->down && !aligned16(gate->down)) return fail(M3_ERR_ALIGN, "gate.down is not 16-byte aligned");
  *gz = gate->z;
  *gw = gate->weight;
  *geps = gate->eps;
  *gdown = gate->down;
  return M3_OK;
}

// BC-normalisation argument checks (bcnorm may be NULL: no normalisation).
int check_bcnorm(const m3_bcnorm* bc, const float** nbw, const float** ncw, float* neps) {
  *nbw = nullptr;
  *ncw = nullptr;
  *neps = 0.f;
  if (!bc) return M3_OK;
  int st;
  if ((st = check_ptr(bc->b_weight, "bcnorm.b_weight")) != M3_OK) return st;
  if ((st = check_ptr(bc->c_weight, "bcnorm.c_weight")) != M3_OK) return st;
  if (!(bc->eps >= 0.f)) return fail(M3_ERR_SHAPE, "bcnorm.eps must be >= 0 (got %g)", (double)bc->eps);
  *nbw = bc->b_weight;
  *ncw = bc->c_weight;
  *neps = bc->eps;
  return M3_OK;
}

int prefill_impl(const m3_dims* dims, int32_t seqlen, const void* x, const void* B, const void* C,
                 const float* dt, const float* lam, const float* theta, const float* A, const float* D,
                 const m3_bcnorm* bcnorm, const m3_gate* gate, bool gated, m3_state* state, void* y,
                 void* workspace, size_t workspace_bytes, void* stream, const char* what,
                 bool noalloc = false) {
  m3::Dims m;
  int st = check_dims(dims, true, &m);
  if (st != M3_OK) return st;
  if (seqlen < 0) return fail(M3_ERR_SHAPE, "seqlen %d < 0", seqlen);
  if ((st = check_state(state, "state")) != M3_OK) return st;
  const void* gz = nullptr;
  const float* gw = nullptr;
  const float* gdown = nullptr;
  float geps = 0.f;
  if (gated) {
    if ((st = check_gate(gate, &gz, &gw, &geps, &gdown)) != M3_OK) return st;
    if (!m3::prefill_pc_path_supported(m))
      return fail(M3_ERR_UNSUPPORTED, "the gated epilogue needs the producer/consumer prefill kernel, whose "
                                      "tiles do not fit for these sizes");
  }
  const float *nbw = nullptr, *ncw = nullptr;
  float neps = 0.f;
  if ((st = check_bcnorm(bcnorm, &nbw, &ncw, &neps)) != M3_OK) return st;
  if (nbw) {
    m3::Dims e = m;
    e.Q = m3::prefill_tile_chunk(m);
    if (!m3::prefill_pc_bcnorm_supported(e))
      return fail(M3_ERR_UNSUPPORTED, "the BC normalisation needs the producer/consumer prefill kernel, whose "
                                      "tiles with the normalisation do not fit for these sizes");
  }
  if (seqlen == 0) return ok();
  m.Q = m3::prefill_tile_chunk(m);
  if ((int64_t)seqlen * m.batch * m.heads * m.R * (m.N > m.P ? m.N : m.P) > ((int64_t)1 << 40))
    return fail(M3_ERR_UNSUPPORTED, "problem too large for 40-bit element offsets");
  if ((int64_t)m.Q * m.heads * m.R * (m.N > m.P ? m.N : m.P) >= ((int64_t)1 << 31))
    return fail(M3_ERR_UNSUPPORTED, "chunk * heads * rank * max(headdim, dstate) must stay below 2^31");
  const void* ptrs[] = {x, B, C, dt, lam, theta, A, D, y};
  const char* names[] = {"x", "B", "C", "dt", "lam", "theta", "A", "D", "y"};
  for (int i = 0; i < 9; ++i)
    if ((st = check_ptr(ptrs[i], names[i])) != M3_OK) return st;
  int nseg = 1, sc = 0;
  plan_segments(m, seqlen, &nseg, &sc);
  const size_t need = workspace_for(m, nseg);
  if (noalloc && need > 0) {
    // the library's own device scratch stands in for the caller's workspace
    if (need > m3::kNoAllocScratchBytes)
      return fail(M3_ERR_UNSUPPORTED, "%s: these sizes need a %zu-byte segment workspace, more than the %zu bytes "
                  "of device scratch; use mamba3_prefill with a caller workspace", what, need,
                  m3::kNoAllocScratchBytes);
    const hipError_t e = m3::noalloc_scratch(&workspace);
    if (e != hipSuccess) return fail(M3_ERR_HIP, "%s: device scratch: %s", what, hipGetErrorString(e));
    workspace_bytes = m3::kNoAllocScratchBytes;
  }
  if (need > 0) {
    if (workspace_bytes < need)
      return fail(M3_ERR_WORKSPACE, "workspace of %zu bytes < required %zu", workspace_bytes, need);
    if ((st = check_ptr(workspace, "workspace")) != M3_OK) return st;
  }
  m3::PrefillArgs a;
  a.x = x;
  a.B = B;
  a.C = C;
  a.dt = dt;
  a.lam = lam;
  a.theta = theta;
  a.A = A;
  a.D = D;
  a.h = state->h;
  a.B_prev = state->B_prev;
  a.x_prev = state->x_prev;
  a.y = y;
  a.disc = m.disc;
  a.gz = gz;
  a.gw = gw;
  a.geps = geps;
  a.gdown = gdown;
  a.nbw = nbw;
  a.ncw = ncw;
  a.neps = neps;
  a.seqlen = seqlen;
  a.nseg = nseg;
  a.seg_chunks = sc;
  a.seg_state = nullptr;
  a.seg_decay = nullptr;
  a.seg_angle = nullptr;
  if (nseg > 1) {
    const size_t cs = (size_t)nseg * m.batch * m.heads;
    char* w = static_cast<char*>(workspace);
    a.seg_state = reinterpret_cast<float*>(w);
    w += align256(cs * m.P * m.N * sizeof(float));
    a.seg_decay = reinterpret_cast<float*>(w);
    w += align256(cs * sizeof(float));
    a.seg_angle = reinterpret_cast<float*>(w);
  }
  return hip_status(m3::launch_prefill(m, a, static_cast<hipStream_t>(stream)), what);
}

int decode_impl(const m3_dims* dims, const void* x, const void* B, const void* C, const float* dt,
                const float* lam, const float* theta, const float* A, const float* D, const m3_bcnorm* bcnorm,
                const m3_gate* gate, bool gated, m3_state* state, void* y, void* stream, const char* what) {
  m3::Dims m;
  int st = check_dims(dims, false, &m);
  if (st != M3_OK) return st;
  if ((st = check_state(state, "state")) != M3_OK) return st;
  const void* gz = nullptr;
  const float* gw = nullptr;
  const float* gdown = nullptr;
  float geps = 0.f;
  if (gated && (st = check_gate(gate, &gz, &gw, &geps, &gdown)) != M3_OK) return st;
  const float *nbw = nullptr, *ncw = nullptr;
  float neps = 0.f;
  if ((st = check_bcnorm(bcnorm, &nbw, &ncw, &neps)) != M3_OK) return st;
  const void* ptrs[] = {x, B, C, dt, lam, theta, A, D, y};
  const char* names[] = {"x", "B", "C", "dt", "lam", "theta", "A", "D", "y"};
  for (int i = 0; i < 9; ++i)
    if ((st = check_ptr(ptrs[i], names[i])) != M3_OK) return st;
  m3::DecodeArgs a;
  a.x = x;
  a.B = B;
  a.C = C;
  a.dt = dt;
  a.lam = lam;
  a.theta = theta;
  a.A = A;
  a.D = D;
  a.h = state->h;
  a.B_prev = state->B_prev;
  a.x_prev = state->x_prev;
  a.y = y;
  a.disc = m.disc;
  a.gz = gz;
  a.gw = gw;
  a.geps = geps;
  a.gdown = gdown;
  a.nbw = nbw;
  a.ncw = ncw;
  a.neps = neps;
  return hip_status(m3::launch_decode(m, a, static_cast<hipStream_t>(stream)), what);
}

}  // namespace

extern "C" {

int mamba3_prefill(const m3_dims* dims, int32_t seqlen, const void* x, const void* B, const void* C,
                   const float* dt, const float* lam, const float* theta, const float* A,
                   const float* D, m3_state* state, void* y, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return prefill_impl(dims, seqlen, x, B, C, dt, lam, theta, A, D, nullptr, nullptr, false, state, y, workspace,
                      workspace_bytes, stream, "mamba3_prefill");
}

int mamba3_prefill_noalloc(const m3_dims* dims, int32_t seqlen, const void* x, const void* B, const void* C,
                           const float* dt, const float* lam, const float* theta, const float* A, const float* D,
                           m3_state* state, void* y, void* stream) {
  return prefill_impl(dims, seqlen, x, B, C, dt, lam, theta, A, D, nullptr, nullptr, false, state, y, nullptr, 0,
                      stream, "mamba3_prefill_noalloc", true);
}

int mamba3_prefill_gated(const m3_dims* dims, int32_t seqlen, const void* x, const void* B, const void* C,
                         const float* dt, const float* lam, const float* theta, const float* A,
                         const float* D, const m3_gate* gate, m3_state* state, void* y, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return prefill_impl(dims, seqlen, x, B, C, dt, lam, theta, A, D, nullptr, gate, true, state, y, workspace,
                      workspace_bytes, stream, "mamba3_prefill_gated");
}

int mamba3_prefill_ex(const m3_dims* dims, int32_t seqlen, const void* x, const void* B, const void* C,
                      const float* dt, const float* lam, const float* theta, const float* A, const float* D,
                      const m3_bcnorm* bcnorm, const m3_gate* gate, m3_state* state, void* y, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return prefill_impl(dims, seqlen, x, B, C, dt, lam, theta, A, D, bcnorm, gate, gate != nullptr, state, y,
                      workspace, workspace_bytes, stream, "mamba3_prefill_ex");
}

int mamba3_decode_step(const m3_dims* dims, const void* x, const void* B, const void* C,
                       const float* dt, const float* lam, const float* theta, const float* A,
                       const float* D, m3_state* state, void* y, void* stream) {
  return decode_impl(dims, x, B, C, dt, lam, theta, A, D, nullptr, nullptr, false, state, y, stream,
                     "mamba3_decode_step");
}

int mamba3_decode_step_gated(const m3_dims* dims, const void* x, const void* B, const void* C,
                             const float* dt, const float* lam, const float* theta, const float* A,
                             const float* D, const m3_gate* gate, m3_state* state, void* y, void* stream) {
  return decode_impl(dims, x, B, C, dt, lam, theta, A, D, nullptr, gate, true, state, y, stream,
                     "mamba3_decode_step_gated");
}

int mamba3_decode_step_ex(const m3_dims* dims, const void* x, const void* B, const void* C, const float* dt,
                          const float* lam, const float* theta, const float* A, const float* D,
                          const m3_bcnorm* bcnorm, const m3_gate* gate, m3_state* state, void* y, void* stream) {
  return decode_impl(dims, x, B, C, dt, lam, theta, A, D, bcnorm, gate, gate != nullptr, state, y, stream,
                     "mamba3_decode_step_ex");
}

int mamba3_prefill_backward_workspace_bytes(const m3_dims* dims, int32_t seqlen, size_t* bytes) {
  m3::Dims m;
  int st = check_dims(dims, false, &m);
  if (st != M3_OK) return st;
  if (!bytes) return fail(M3_ERR_NULL, "bytes is NULL");
  if (seqlen < 0) return fail(M3_ERR_SHAPE, "seqlen %d < 0", seqlen);
  if (!m3::backward_supported(m))
    return fail(M3_ERR_UNSUPPORTED, "the backward pass needs R in {1, 2, 4}, headdim and dstate multiples of 16 "
                "with headdim * dstate <= 8192 (got R %d, %d x %d)", m.R, m.P, m.N);
  *bytes = seqlen > 0 ? m3::backward_workspace_bytes(m, seqlen) : 0;
  return ok();
}

int mamba3_prefill_backward(const m3_dims* dims, int32_t seqlen, const void* x, const void* B, const void* C,
                            const float* dt, const float* lam, const float* theta, const float* A,
                            const float* D, const m3_state* state0, const void* dy, const float* dh_final,
                            const m3_grads* grads, void* workspace, size_t workspace_bytes, void* stream) {
  m3::Dims m;
  int st = check_dims(dims, false, &m);
  if (st != M3_OK) return st;
  if (seqlen < 0) return fail(M3_ERR_SHAPE, "seqlen %d < 0", seqlen);
  if (!m3::backward_supported(m))
    return fail(M3_ERR_UNSUPPORTED, "the backward pass needs R in {1, 2, 4}, headdim and dstate multiples of 16 "
                "with headdim * dstate <= 8192 (got R %d, %d x %d)", m.R, m.P, m.N);
  if (!state0) return fail(M3_ERR_NULL, "state0 is NULL");
  if ((st = check_ptr(state0->h, "state0.h")) != M3_OK) return st;
  if ((st = check_ptr(state0->B_prev, "state0.B_prev")) != M3_OK) return st;
  if ((st = check_ptr(state0->x_prev, "state0.x_prev")) != M3_OK) return st;
  if (!grads) return fail(M3_ERR_NULL, "grads is NULL");
  const void* gp[] = {grads->dx, grads->dB, grads->dC, grads->ddt, grads->dlam, grads->dtheta,
                      grads->dA, grads->dD, grads->dh0, grads->dB_prev, grads->dx_prev};
  const char* gn[] = {"grads.dx", "grads.dB", "grads.dC", "grads.ddt", "grads.dlam", "grads.dtheta",
                      "grads.dA", "grads.dD", "grads.dh0", "grads.dB_prev", "grads.dx_prev"};
  for (int i = 0; i < 11; ++i)
    if ((st = check_ptr(gp[i], gn[i])) != M3_OK) return st;
  if (dh_final && (st = check_ptr(dh_final, "dh_final")) != M3_OK) return st;
  if (seqlen == 0) return fail(M3_ERR_SHAPE, "seqlen 0: there is nothing to differentiate");
  const void* ptrs[] = {x, B, C, dt, lam, theta, A, D, dy};
  const char* names[] = {"x", "B", "C", "dt", "lam", "theta", "A", "D", "dy"};
  for (int i = 0; i < 9; ++i)
    if ((st = check_ptr(ptrs[i], names[i])) != M3_OK) return st;
  const size_t need = m3::backward_workspace_bytes(m, seqlen);
  if (workspace_bytes < need)
    return fail(M3_ERR_WORKSPACE, "workspace of %zu bytes < required %zu", workspace_bytes, need);
  if ((st = check_ptr(workspace, "workspace")) != M3_OK) return st;
  m3::BackwardArgs a;
  a.x = x;
  a.B = B;
  a.C = C;
  a.dt = dt;
  a.lam = lam;
  a.theta = theta;
  a.A = A;
  a.D = D;
  a.h = state0->h;
  a.B_prev = state0->B_prev;
  a.x_prev = state0->x_prev;
  a.dy = dy;
  a.dh_final = dh_final;
  a.dx = grads->dx;
  a.dB = grads->dB;
  a.dC = grads->dC;
  a.ddt = grads->ddt;
  a.dlam = grads->dlam;
  a.dtheta = grads->dtheta;
  a.dA = grads->dA;
  a.dD = grads->dD;
  a.dh0 = grads->dh0;
  a.dB_prev = grads->dB_prev;
  a.dx_prev = grads->dx_prev;
  a.ws = workspace;
  a.seqlen = seqlen;
  a.disc = m.disc;
  return hip_status(m3::launch_backward(m, a, static_cast<hipStream_t>(stream)), "mamba3_prefill_backward");
}

}  // extern "C"

