/* Drives every entry point of include/mamba3.h through its host-side checks
 * (NULL, shape, dtype, alignment, unsupported size, short workspace) and
 * through to the launch, which the host stubs refuse (M3_ERR_HIP), so that a
 * sanitizer build of the validation layer sees every path.  Compiled as C, so
 * the header is also checked to be valid C.  Prints "ok <n> checks" and
 * exits 0 when every status is the documented one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mamba3.h"

static int n_checks = 0, n_fail = 0;

static void expect(int got, int want, const char* what) {
  ++n_checks;
  if (got != want) {
    ++n_fail;
    fprintf(stderr, "FAIL %s: got %d want %d (%s)\n", what, got, want, m3_last_error());
  } else if (want < 0 && strlen(m3_last_error()) == 0) {
    ++n_fail;
    fprintf(stderr, "FAIL %s: no message\n", what);
  }
}

static m3_dims dims(int P, int N, int R, int Q, int io) {
  m3_dims d;
  memset(&d, 0, sizeof d);
  d.batch = 2;
  d.heads = 3;
  d.headdim = P;
  d.dstate = N;
  d.rank = R;
  d.chunk = Q;
  d.io_dtype = io;
  d.disc = M3_DISC_EXP_TRAPEZOID;
  return d;
}

int main(void) {
  /* 16-byte aligned fake device addresses: never dereferenced on the host */
  void* const F = (void*)(uintptr_t)0x10000;
  void* const MIS = (void*)(uintptr_t)0x10004;
  float* const FF = (float*)F;
  m3_state st = {FF, F, F};
  m3_dims d = dims(64, 128, 1, 64, M3_BF16);
  size_t hb = 0, bb = 0, xb = 0, ws = 0;

  expect(m3_abi_version(), M3_ABI_VERSION, "abi version");
  expect(m3_state_bytes(&d, &hb, &bb, &xb), M3_OK, "state_bytes");
  expect(hb == (size_t)2 * 3 * 64 * 128 * 4 ? M3_OK : -99, M3_OK, "state_bytes h");
  expect(m3_state_bytes(NULL, &hb, NULL, NULL), M3_ERR_NULL, "state_bytes NULL dims");

  /* every dims field out of range */
  {
    m3_dims e = d; e.batch = 0; expect(m3_state_bytes(&e, &hb, NULL, NULL), M3_ERR_SHAPE, "batch 0");
    e = d; e.dstate = 15; expect(mamba3_prefill_workspace_bytes(&e, 16, &ws), M3_ERR_UNSUPPORTED, "odd N");
    e = d; e.io_dtype = 9; expect(mamba3_prefill_workspace_bytes(&e, 16, &ws), M3_ERR_DTYPE, "dtype");
    e = d; e.disc = 3; expect(mamba3_prefill_workspace_bytes(&e, 16, &ws), M3_ERR_UNSUPPORTED, "disc");
    e = d; e.rank = 9; expect(mamba3_prefill_workspace_bytes(&e, 16, &ws), M3_ERR_UNSUPPORTED, "rank 9");
    e = d; e.chunk = 0; expect(mamba3_prefill_workspace_bytes(&e, 16, &ws), M3_ERR_SHAPE, "chunk 0");
    e = d; e.heads = 1 << 22; expect(mamba3_prefill_workspace_bytes(&e, 16, &ws), M3_ERR_UNSUPPORTED, "too many");
  }
  expect(mamba3_prefill_workspace_bytes(&d, -1, &ws), M3_ERR_SHAPE, "seqlen < 0");
  expect(mamba3_prefill_workspace_bytes(&d, 16, NULL), M3_ERR_NULL, "ws NULL");

  /* state calls */
  expect(m3_state_zero(&d, &st, NULL), M3_ERR_HIP, "state_zero launch");
  expect(m3_state_zero(&d, NULL, NULL), M3_ERR_NULL, "state_zero NULL");
  {
    m3_state bad = {FF, MIS, F};
    expect(m3_state_zero(&d, &bad, NULL), M3_ERR_ALIGN, "state misaligned");
  }
  expect(m3_state_load(&d, &st, FF, F, F, NULL), M3_ERR_HIP, "state_load launch");
  expect(m3_state_load(&d, &st, NULL, F, F, NULL), M3_ERR_NULL, "state_load NULL h");
  expect(m3_state_readout(&d, &st, FF, F, MIS, NULL), M3_ERR_ALIGN, "readout misaligned");

  /* prefill: each pointer NULL and misaligned, then the launch */
  {
    const void* p[9];
    for (int i = 0; i < 10; ++i) {
      for (int k = 0; k < 9; ++k) p[k] = F;
      if (i < 9) p[i] = NULL;
      int s = mamba3_prefill(&d, 16, p[0], p[1], p[2], (const float*)p[3], (const float*)p[4], (const float*)p[5],
                             (const float*)p[6], (const float*)p[7], &st, (void*)p[8], NULL, 0, NULL);
      expect(s, i < 9 ? M3_ERR_NULL : M3_ERR_HIP, "prefill pointer");
    }
    for (int i = 0; i < 9; ++i) {
      for (int k = 0; k < 9; ++k) p[k] = F;
      p[i] = MIS;
      int s = mamba3_prefill(&d, 16, p[0], p[1], p[2], (const float*)p[3], (const float*)p[4], (const float*)p[5],
                             (const float*)p[6], (const float*)p[7], &st, (void*)p[8], NULL, 0, NULL);
      expect(s, M3_ERR_ALIGN, "prefill misaligned");
    }
  }
  expect(mamba3_prefill(&d, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, &st, NULL, NULL, 0, NULL), M3_OK,
         "prefill seqlen 0");
  /* few long chains: the segment path needs a workspace */
  {
    m3_dims e = dims(64, 128, 1, 64, M3_BF16);
    e.batch = 1;
    e.heads = 2;
    const int T = 64 * 40;
    expect(mamba3_prefill_workspace_bytes(&e, T, &ws), M3_OK, "segment ws");
    expect(ws > 0 ? M3_OK : -99, M3_OK, "segment ws > 0");
    expect(mamba3_prefill(&e, T, F, F, F, FF, FF, FF, FF, FF, &st, F, F, ws - 1, NULL), M3_ERR_WORKSPACE,
           "short ws");
    expect(mamba3_prefill(&e, T, F, F, F, FF, FF, FF, FF, FF, &st, F, NULL, ws, NULL), M3_ERR_NULL, "ws NULL");
    expect(mamba3_prefill(&e, T, F, F, F, FF, FF, FF, FF, FF, &st, F, F, ws, NULL), M3_ERR_HIP, "segment launch");
    expect(mamba3_prefill_noalloc(&e, T, F, F, F, FF, FF, FF, FF, FF, &st, F, NULL), M3_ERR_HIP, "noalloc launch");
    e.heads = 64;
    e.headdim = 128;
    expect(mamba3_prefill_noalloc(&e, 1 << 16, F, F, F, FF, FF, FF, FF, FF, &st, F, NULL), M3_ERR_UNSUPPORTED,
           "noalloc beyond scratch");
  }

  /* gate and BC norm arguments */
  {
    m3_gate g = {F, FF, 1e-5f, NULL};
    expect(mamba3_prefill_gated(&d, 16, F, F, F, FF, FF, FF, FF, FF, &g, &st, F, NULL, 0, NULL), M3_ERR_HIP, "gated");
    g.eps = -1.f;
    expect(mamba3_prefill_gated(&d, 16, F, F, F, FF, FF, FF, FF, FF, &g, &st, F, NULL, 0, NULL), M3_ERR_SHAPE,
           "gated eps");
    g.eps = 1e-5f;
    g.down = (const float*)MIS;
    expect(mamba3_decode_step_gated(&d, F, F, F, FF, FF, FF, FF, FF, &g, &st, F, NULL), M3_ERR_ALIGN, "down align");
    expect(mamba3_prefill_gated(&d, 16, F, F, F, FF, FF, FF, FF, FF, NULL, &st, F, NULL, 0, NULL), M3_ERR_NULL,
           "gate NULL");
    m3_bcnorm bc = {FF, NULL, 1e-6f};
    expect(mamba3_prefill_ex(&d, 16, F, F, F, FF, FF, FF, FF, FF, &bc, NULL, &st, F, NULL, 0, NULL), M3_ERR_NULL,
           "bcnorm NULL");
    bc.c_weight = FF;
    expect(mamba3_prefill_ex(&d, 16, F, F, F, FF, FF, FF, FF, FF, &bc, NULL, &st, F, NULL, 0, NULL), M3_ERR_HIP,
           "bcnorm launch");
    expect(mamba3_decode_step_ex(&d, F, F, F, FF, FF, FF, FF, FF, &bc, NULL, &st, F, NULL), M3_ERR_HIP, "dec ex");
  }

  /* decode */
  expect(mamba3_decode_step(&d, F, F, F, FF, FF, FF, FF, FF, &st, F, NULL), M3_ERR_HIP, "decode launch");
  expect(mamba3_decode_step(&d, F, F, F, FF, FF, NULL, FF, FF, &st, F, NULL), M3_ERR_NULL, "decode NULL");

  /* backward */
  {
    m3_grads g = {FF, FF, FF, FF, FF, FF, FF, FF, FF, FF, FF};
    m3_dims e = dims(64, 128, 1, 64, M3_BF16);
    expect(mamba3_prefill_backward_workspace_bytes(&e, 100, &ws), M3_OK, "bwd ws");
    expect(mamba3_prefill_backward(&e, 100, F, F, F, FF, FF, FF, FF, FF, &st, F, NULL, &g, F, ws - 1, NULL),
           M3_ERR_WORKSPACE, "bwd short ws");
    expect(mamba3_prefill_backward(&e, 100, F, F, F, FF, FF, FF, FF, FF, &st, F, NULL, &g, F, ws, NULL), M3_ERR_HIP,
           "bwd launch");
    expect(mamba3_prefill_backward(&e, 0, F, F, F, FF, FF, FF, FF, FF, &st, F, NULL, &g, F, ws, NULL), M3_ERR_SHAPE,
           "bwd seqlen 0");
    g.dtheta = NULL;
    expect(mamba3_prefill_backward(&e, 100, F, F, F, FF, FF, FF, FF, FF, &st, F, NULL, &g, F, ws, NULL), M3_ERR_NULL,
           "bwd grads NULL");
    e.rank = 3;
    expect(mamba3_prefill_backward_workspace_bytes(&e, 100, &ws), M3_ERR_UNSUPPORTED, "bwd rank 3");
  }

  /* a long message does not overrun the library's error buffer */
  {
    m3_dims e = dims(48, 100000, 7, 64, M3_BF16);
    expect(mamba3_prefill_workspace_bytes(&e, 16, &ws), M3_ERR_UNSUPPORTED, "long message");
  }
  if (n_fail) {
    fprintf(stderr, "%d of %d checks failed\n", n_fail, n_checks);
    return 1;
  }
  printf("ok %d checks\n", n_checks);
  return 0;
}
