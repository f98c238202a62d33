/*
 * Argument validation of every entry point of include/attn_jvp.h, from plain
 * C: each call below passes an invalid argument (a NULL or misaligned pointer,
 * a size out of range, a bad scale, workspace or dtype) and must return the
 * documented error code before anything is launched.  The pointers are fake
 * device addresses that are never dereferenced, so this runs without a GPU.
 * Built twice by __graft_entry__.build(): plainly, and with the C ABI's host
 * code under AddressSanitizer and UndefinedBehaviorSanitizer (the size
 * arithmetic of the validation, e.g. products of B, H, N and d, must not
 * overflow).  Prints one line per failed check; exit status 0 when all pass.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "attn_jvp.h"

static int failures = 0, checks = 0;

static void expect(const char *what, int got, int want) {
  ++checks;
  if (got != want) {
    printf("FAIL %s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

/* fake, 256-byte aligned device addresses (never dereferenced) */
#define P(i) ((void *)(uintptr_t)(0x7F0000000000ull + (uint64_t)(i) * 0x100000ull))
#define F(i) ((float *)P(i))
#define MIS(i) ((void *)((char *)P(i) + 8))

typedef int (*fwd_fn)(const void *, const void *, const void *, const void *, const void *,
                      const void *, float *, float *, float *, int, int, int, int, int, float,
                      attn_jvp_stream_t);

static int call_f32(const void *q, const void *k, const void *v, const void *tq, const void *tk,
                    const void *tv, float *o, float *to, float *lse, int B, int H, int Nq,
                    int Nk, int d, float s, attn_jvp_stream_t st) {
  return attn_jvp_fwd_f32((const float *)q, (const float *)k, (const float *)v,
                          (const float *)tq, (const float *)tk, (const float *)tv, o, to, lse, B,
                          H, Nq, Nk, d, s, st);
}

static int call_ws(const void *q, const void *k, const void *v, const void *tq, const void *tk,
                   const void *tv, float *o, float *to, float *lse, int B, int H, int Nq, int Nk,
                   int d, float s, attn_jvp_stream_t st) {
  return attn_jvp_fwd_ws(q, k, v, tq, tk, tv, o, to, lse, B, H, Nq, Nk, d, s, P(20),
                         (size_t)1 << 60, st);
}

/* the checks shared by the four forward entry points with the full signature */
static void forward_family(const char *name, fwd_fn f) {
  char what[128];
  void *p[8];
  for (int i = 0; i < 8; ++i) p[i] = P(i);
  for (int i = 0; i < 8; ++i) {
    void *q[8];
    memcpy(q, p, sizeof q);
    q[i] = NULL;
    snprintf(what, sizeof what, "%s NULL pointer %d", name, i);
    expect(what, f(q[0], q[1], q[2], q[3], q[4], q[5], (float *)q[6], (float *)q[7], NULL, 1, 1,
                   4, 4, 128, 0.1f, NULL),
           ATTN_JVP_EINVAL);
  }
  for (int i = 0; i < 8; ++i) {
    void *q[8];
    memcpy(q, p, sizeof q);
    q[i] = MIS(i);
    snprintf(what, sizeof what, "%s misaligned pointer %d", name, i);
    expect(what, f(q[0], q[1], q[2], q[3], q[4], q[5], (float *)q[6], (float *)q[7], NULL, 1, 1,
                   4, 4, 128, 0.1f, NULL),
           ATTN_JVP_EALIGN);
  }
  const int sizes[][4] = {{0, 1, 4, 4}, {1, 0, 4, 4}, {1, 1, 0, 4}, {1, 1, 4, 0},
                          {-1, 1, 4, 4}, {1, -7, 4, 4}, {1, 1, -4, 4}, {1, 1, 4, -2147483647 - 1}};
  for (int i = 0; i < 8; ++i) {
    snprintf(what, sizeof what, "%s size %d", name, i);
    expect(what, f(p[0], p[1], p[2], p[3], p[4], p[5], F(6), F(7), NULL, sizes[i][0], sizes[i][1],
                   sizes[i][2], sizes[i][3], 128, 0.1f, NULL),
           ATTN_JVP_EINVAL);
  }
  snprintf(what, sizeof what, "%s d = 96", name);
  expect(what, f(p[0], p[1], p[2], p[3], p[4], p[5], F(6), F(7), NULL, 1, 1, 4, 4, 96, 0.1f, NULL),
         ATTN_JVP_EUNSUPPORTED);
  snprintf(what, sizeof what, "%s one slice past 2^31 bytes", name);
  expect(what, f(p[0], p[1], p[2], p[3], p[4], p[5], F(6), F(7), NULL, 1, 1, 4, 1 << 30, 128,
                 0.1f, NULL),
         ATTN_JVP_EUNSUPPORTED);
  expect(what, f(p[0], p[1], p[2], p[3], p[4], p[5], F(6), F(7), NULL, 1, 1, 2147483647, 4, 128,
                 0.1f, NULL),
         ATTN_JVP_EUNSUPPORTED);
  snprintf(what, sizeof what, "%s B*H past 2^31 - 1", name);
  expect(what, f(p[0], p[1], p[2], p[3], p[4], p[5], F(6), F(7), NULL, 65536, 65536, 4, 4, 128,
                 0.1f, NULL),
         ATTN_JVP_EUNSUPPORTED);
  const float bad[3] = {NAN, INFINITY, -INFINITY};
  for (int i = 0; i < 3; ++i) {
    snprintf(what, sizeof what, "%s bad scale %d", name, i);
    expect(what, f(p[0], p[1], p[2], p[3], p[4], p[5], F(6), F(7), NULL, 1, 1, 4, 4, 128, bad[i],
                   NULL),
           ATTN_JVP_EINVAL);
  }
  snprintf(what, sizeof what, "%s misaligned lse", name);
  expect(what, f(p[0], p[1], p[2], p[3], p[4], p[5], F(6), F(7), (float *)((char *)P(8) + 2), 1, 1,
                 4, 4, 128, 0.1f, NULL),
         ATTN_JVP_EALIGN);
}

int main(void) {
  /* the fake pointers must never reach a device: with a GPU visible, a check
     that wrongly passed validation would launch on them */
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    printf("skipped: a GPU is visible (this program runs on hosts without one)\n");
    return 0;
  }
  forward_family("attn_jvp_fwd", attn_jvp_fwd);
  forward_family("attn_jvp_fwd_ws", call_ws);
  forward_family("attn_jvp_fwd_noalloc", attn_jvp_fwd_noalloc);
  forward_family("attn_jvp_fwd_f32", call_f32);

  /* the workspace of attn_jvp_fwd_ws */
  const size_t need = attn_jvp_workspace_bytes(1, 2, 100, 128);
  expect("workspace bytes > 0", need > 0, 1);
  expect("ws NULL", attn_jvp_fwd_ws(P(0), P(1), P(2), P(3), P(4), P(5), F(6), F(7), NULL, 1, 2, 4,
                                    100, 128, 0.1f, NULL, need, NULL),
         ATTN_JVP_EINVAL);
  expect("ws short", attn_jvp_fwd_ws(P(0), P(1), P(2), P(3), P(4), P(5), F(6), F(7), NULL, 1, 2, 4,
                                     100, 128, 0.1f, P(9), need - 1, NULL),
         ATTN_JVP_EINVAL);
  expect("ws misaligned", attn_jvp_fwd_ws(P(0), P(1), P(2), P(3), P(4), P(5), F(6), F(7), NULL, 1,
                                          2, 4, 100, 128, 0.1f, (char *)P(9) + 16, need, NULL),
         ATTN_JVP_EALIGN);
  expect("noalloc: one slice past its buffer",
         attn_jvp_fwd_noalloc(P(0), P(1), P(2), P(3), P(4), P(5), F(6), F(7), NULL, 1, 1, 4,
                              131072, 128, 0.1f, NULL),
         ATTN_JVP_EUNSUPPORTED);

  /* workspace sizes of invalid calls are 0 */
  expect("workspace_bytes B = 0", attn_jvp_workspace_bytes(0, 1, 4, 128) == 0, 1);
  expect("workspace_bytes d = 96", attn_jvp_workspace_bytes(1, 1, 4, 96) == 0, 1);
  expect("workspace_bytes Nk < 0", attn_jvp_workspace_bytes(1, 1, -4, 128) == 0, 1);
  expect("splitkv bytes nsplit < 0", attn_jvp_splitkv_workspace_bytes(1, 1, 4, 4, 128, -1) == 0, 1);
  expect("splitkv bytes huge Nk", attn_jvp_splitkv_workspace_bytes(1, 1, 4, 1 << 30, 128, 0) == 0, 1);
  expect("bwd bytes H = 0", attn_bwd_workspace_bytes(1, 0, 4, 4, 128) == 0, 1);

  /* the two phases */
  expect("pack_kv NULL tv", attn_jvp_pack_kv(P(0), P(1), P(2), NULL, 1, 1, 100, 128, P(9), need,
                                             NULL),
         ATTN_JVP_EINVAL);
  expect("pack_kv short ws", attn_jvp_pack_kv(P(0), P(1), P(2), P(3), 1, 2, 100, 128, P(9),
                                              need - 256, NULL),
         ATTN_JVP_EINVAL);
  expect("pack_kv misaligned k", attn_jvp_pack_kv(MIS(0), P(1), P(2), P(3), 1, 2, 100, 128, P(9),
                                                  need, NULL),
         ATTN_JVP_EALIGN);
  expect("fwd_packed NULL tq", attn_jvp_fwd_packed(P(0), NULL, P(9), need, F(6), F(7), NULL, 1, 2,
                                                   4, 100, 128, 0.1f, NULL),
         ATTN_JVP_EINVAL);
  expect("fwd_packed bad scale", attn_jvp_fwd_packed(P(0), P(1), P(9), need, F(6), F(7), NULL, 1,
                                                     2, 4, 100, 128, NAN, NULL),
         ATTN_JVP_EINVAL);

  /* extended form, split-KV and the forward pass */
  expect("fwd_ex bad out_dtype", attn_jvp_fwd_ex(P(0), P(1), P(2), NULL, NULL, NULL, P(6), P(7),
                                                 NULL, NULL, 1, 1, 4, 4, 128, 0.1f, 7, NULL, 0,
                                                 NULL),
         ATTN_JVP_EINVAL);
  expect("fwd_ex misaligned tangent", attn_jvp_fwd_ex(P(0), P(1), P(2), MIS(3), NULL, NULL, P(6),
                                                      P(7), NULL, NULL, 1, 1, 4, 4, 128, 0.1f, 0,
                                                      NULL, 0, NULL),
         ATTN_JVP_EALIGN);
  expect("fwd_ex misaligned tlse", attn_jvp_fwd_ex(P(0), P(1), P(2), NULL, NULL, NULL, P(6), P(7),
                                                   NULL, (float *)((char *)P(8) + 1), 1, 1, 4, 4,
                                                   128, 0.1f, 0, NULL, 0, NULL),
         ATTN_JVP_EALIGN);
  expect("splitkv nsplit < 0", attn_jvp_fwd_splitkv(P(0), P(1), P(2), NULL, NULL, NULL, F(6), F(7),
                                                    NULL, NULL, 1, 1, 4, 4, 128, 0.1f, -1, NULL, 0,
                                                    NULL),
         ATTN_JVP_EINVAL);
  expect("fwd_splitkv NULL o", attn_fwd_splitkv(P(0), P(1), P(2), NULL, NULL, 1, 1, 4, 4, 128,
                                                0.1f, 0, NULL, 0, NULL),
         ATTN_JVP_EINVAL);
  expect("attn_fwd NULL v", attn_fwd(P(0), P(1), NULL, P(6), NULL, 1, 1, 4, 4, 128, 0.1f, 0, NULL,
                                     0, NULL),
         ATTN_JVP_EINVAL);
  expect("attn_fwd bad out_dtype", attn_fwd(P(0), P(1), P(2), P(6), NULL, 1, 1, 4, 4, 128, 0.1f,
                                            -1, NULL, 0, NULL),
         ATTN_JVP_EINVAL);

  /* merge */
  expect("merge P = 0", attn_jvp_merge(F(0), F(1), NULL, NULL, 0, 4, 128, F(2), F(3), NULL, NULL,
                                       NULL),
         ATTN_JVP_EINVAL);
  expect("merge P > 1024", attn_jvp_merge(F(0), F(1), NULL, NULL, 1025, 4, 128, F(2), F(3), NULL,
                                          NULL, NULL),
         ATTN_JVP_EUNSUPPORTED);
  expect("merge half a tangent", attn_jvp_merge(F(0), F(1), F(4), NULL, 2, 4, 128, F(2), F(3), F(5),
                                                NULL, NULL),
         ATTN_JVP_EINVAL);
  expect("merge d = 32", attn_jvp_merge(F(0), F(1), NULL, NULL, 2, 4, 32, F(2), F(3), NULL, NULL,
                                        NULL),
         ATTN_JVP_EUNSUPPORTED);

  /* backward */
  expect("bwd NULL go", attn_bwd(P(0), P(1), P(2), F(3), NULL, F(5), F(6), F(7), F(8), 1, 1, 4, 4,
                                 128, 0.1f, NULL, 0, NULL),
         ATTN_JVP_EINVAL);
  expect("bwd misaligned lse", attn_bwd(P(0), P(1), P(2), F(3), P(4), (float *)((char *)P(5) + 2),
                                        F(6), F(7), F(8), 1, 1, 4, 4, 128, 0.1f, NULL, 0, NULL),
         ATTN_JVP_EALIGN);
  expect("bwd short ws", attn_bwd(P(0), P(1), P(2), F(3), P(4), F(5), F(6), F(7), F(8), 1, 1, 4, 4,
                                  128, 0.1f, P(9), 16, NULL),
         ATTN_JVP_EINVAL);

  /* every status has a name */
  const int codes[6] = {ATTN_JVP_OK, ATTN_JVP_EINVAL, ATTN_JVP_EUNSUPPORTED, ATTN_JVP_EALIGN,
                        ATTN_JVP_ELAUNCH, 12345};
  for (int i = 0; i < 6; ++i) expect("strerror non-empty", attn_jvp_strerror(codes[i])[0] != 0, 1);

  printf("%d validation checks, %d failed\n", checks, failures);
  if (!failures) printf("validation checks passed\n");
  return failures ? 1 : 0;
}
