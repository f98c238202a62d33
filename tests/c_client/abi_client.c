/*
 * A plain C client of the library (no Python, no torch): device buffers from
 * the HIP runtime, inputs from a fixed-seed generator, and checks of results
 * whose values follow from the definition of attention and its JVP alone
 * (softmax attention, O = softmax(s Q K^T) V, and its directional derivative;
 * the rCM record in the Anthology of the SOTA, "Key takeaways", "JVP at
 * production scale"):
 *   one key      P = 1, so O = v0, dO = dv0 and lse = s q.k0 (V, dV pass
 *                through fp16 in the kernel: exact for these values but the
 *                rare ones below 2^-14);
 *   Q = dQ = 0   uniform attention: O = mean_j v_j, lse = ln Nk, and with
 *                dK = 0 the scores do not move, so dO = mean_j dv_j;
 * plus the bf16 and fp32 entry points agreeing on random inputs, and argument
 * errors returned before any launch.  Prints one line per check; exit status 0
 * when all pass.  With the argument --no-gpu only the argument errors are
 * checked (they return before touching a device).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "attn_jvp.h"

static int failures = 0;

static void report(const char *what, int ok, double err) {
  printf("%-52s %s (%.3e)\n", what, ok ? "ok" : "FAIL", err);
  if (!ok) ++failures;
}

/* splitmix64, for reproducible inputs */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return (double)(z >> 11) / 9007199254740992.0;
}
static double normal(void) {
  double u = uniform(), v = uniform();
  if (u < 1e-300) u = 1e-300;
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

/* bf16 <-> float (round to nearest even) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

#define CHECK_HIP(x)                                                     \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      printf("HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__);   \
      exit(2);                                                           \
    }                                                                    \
  } while (0)

static void *dev_copy(const void *host, size_t bytes) {
  void *p = NULL;
  CHECK_HIP(hipMalloc(&p, bytes));
  CHECK_HIP(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
  return p;
}

/* one (b, h) slice: B = H = 1 */
typedef struct {
  int nq, nk, d;
  uint16_t *q, *k, *v, *tq, *tk, *tv; /* host bf16 */
} Case;

static uint16_t *fill(int n, double sigma, int zero) {
  uint16_t *x = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n);
  for (int i = 0; i < n; ++i) x[i] = zero ? 0 : to_bf16((float)(sigma * normal()));
  return x;
}

/* run attn_jvp_fwd; returns host fp32 O, dO, lse in one buffer */
static float *run_bf16(const Case *c, float scale, int *rc) {
  const size_t nq = (size_t)c->nq * c->d, nk = (size_t)c->nk * c->d;
  void *q = dev_copy(c->q, nq * 2), *tq = dev_copy(c->tq, nq * 2);
  void *k = dev_copy(c->k, nk * 2), *v = dev_copy(c->v, nk * 2);
  void *tk = dev_copy(c->tk, nk * 2), *tv = dev_copy(c->tv, nk * 2);
  float *o, *to, *lse;
  CHECK_HIP(hipMalloc((void **)&o, nq * 4));
  CHECK_HIP(hipMalloc((void **)&to, nq * 4));
  CHECK_HIP(hipMalloc((void **)&lse, (size_t)c->nq * 4));
  *rc = attn_jvp_fwd(q, k, v, tq, tk, tv, o, to, lse, 1, 1, c->nq, c->nk, c->d, scale, NULL);
  CHECK_HIP(hipDeviceSynchronize());
  float *out = (float *)malloc((2 * nq + c->nq) * 4);
  CHECK_HIP(hipMemcpy(out, o, nq * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out + nq, to, nq * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out + 2 * nq, lse, (size_t)c->nq * 4, hipMemcpyDeviceToHost));
  void *bufs[9] = {q, tq, k, v, tk, tv, o, to, lse};
  for (int i = 0; i < 9; ++i) CHECK_HIP(hipFree(bufs[i]));
  return out;
}

static void one_key(void) {
  Case c = {77, 1, 128, 0, 0, 0, 0, 0, 0};
  c.q = fill(c.nq * c.d, 1.0, 0), c.k = fill(c.d, 1.0, 0), c.v = fill(c.d, 1.0, 0);
  c.tq = fill(c.nq * c.d, 0.1, 0), c.tk = fill(c.d, 0.1, 0), c.tv = fill(c.d, 0.1, 0);
  const float s = 0.2f;
  int rc;
  float *out = run_bf16(&c, s, &rc);
  report("one key: status", rc == ATTN_JVP_OK, (double)rc);
  double eo = 0, edo = 0, el = 0;
  for (int i = 0; i < c.nq; ++i) {
    double qk = 0;
    for (int j = 0; j < c.d; ++j) {
      eo = fmax(eo, fabs(out[i * c.d + j] - from_bf16(c.v[j])));
      edo = fmax(edo, fabs(out[c.nq * c.d + i * c.d + j] - from_bf16(c.tv[j])));
      qk += from_bf16(c.q[i * c.d + j]) * from_bf16(c.k[j]);
    }
    el = fmax(el, fabs(out[2 * c.nq * c.d + i] - s * qk));
  }
  report("one key: O = v0", eo <= 1e-6, eo);
  report("one key: dO = dv0", edo <= 1e-5, edo);
  report("one key: lse = s q.k0", el <= 1e-4, el);
  free(out);
}

static void uniform_attention(void) {
  Case c = {300, 517, 64, 0, 0, 0, 0, 0, 0};
  c.q = fill(c.nq * c.d, 1.0, 1), c.k = fill(c.nk * c.d, 1.0, 0), c.v = fill(c.nk * c.d, 1.0, 0);
  c.tq = fill(c.nq * c.d, 0.1, 1), c.tk = fill(c.nk * c.d, 0.1, 1), c.tv = fill(c.nk * c.d, 0.1, 0);
  int rc;
  float *out = run_bf16(&c, 0.125f, &rc);
  report("uniform attention: status", rc == ATTN_JVP_OK, (double)rc);
  double eo = 0, edo = 0, el = 0;
  for (int j = 0; j < c.d; ++j) {
    double mv = 0, mdv = 0;
    for (int r = 0; r < c.nk; ++r) {
      mv += from_bf16(c.v[r * c.d + j]);
      mdv += from_bf16(c.tv[r * c.d + j]);
    }
    mv /= c.nk, mdv /= c.nk;
    for (int i = 0; i < c.nq; ++i) {
      eo = fmax(eo, fabs(out[i * c.d + j] - mv));
      edo = fmax(edo, fabs(out[c.nq * c.d + i * c.d + j] - mdv));
    }
  }
  for (int i = 0; i < c.nq; ++i) el = fmax(el, fabs(out[2 * c.nq * c.d + i] - log((double)c.nk)));
  report("uniform attention: O = mean of V rows", eo <= 1e-5, eo);
  report("uniform attention: dO = mean of dV rows", edo <= 1e-5, edo);
  report("uniform attention: lse = ln Nk", el <= 1e-5, el);
  free(out);
}

static void bf16_vs_fp32(void) {
  Case c = {333, 271, 128, 0, 0, 0, 0, 0, 0};
  c.q = fill(c.nq * c.d, 1.0, 0), c.k = fill(c.nk * c.d, 1.0, 0), c.v = fill(c.nk * c.d, 1.0, 0);
  c.tq = fill(c.nq * c.d, 0.1, 0), c.tk = fill(c.nk * c.d, 0.1, 0), c.tv = fill(c.nk * c.d, 0.1, 0);
  const float s = 0.08838834764831843f;
  int rc;
  float *b = run_bf16(&c, s, &rc);
  /* the same (bf16-exact) values as fp32 inputs */
  const size_t nq = (size_t)c.nq * c.d, nk = (size_t)c.nk * c.d;
  float *h[6];
  const uint16_t *src[6] = {c.q, c.k, c.v, c.tq, c.tk, c.tv};
  const size_t n[6] = {nq, nk, nk, nq, nk, nk};
  void *dv[6];
  for (int t = 0; t < 6; ++t) {
    h[t] = (float *)malloc(n[t] * 4);
    for (size_t i = 0; i < n[t]; ++i) h[t][i] = (float)from_bf16(src[t][i]);
    dv[t] = dev_copy(h[t], n[t] * 4);
  }
  float *o, *to;
  CHECK_HIP(hipMalloc((void **)&o, nq * 4));
  CHECK_HIP(hipMalloc((void **)&to, nq * 4));
  int rc2 = attn_jvp_fwd_f32((const float *)dv[0], (const float *)dv[1], (const float *)dv[2],
                             (const float *)dv[3], (const float *)dv[4], (const float *)dv[5], o, to,
                             NULL, 1, 1, c.nq, c.nk, c.d, s, NULL);
  CHECK_HIP(hipDeviceSynchronize());
  float *f = (float *)malloc(2 * nq * 4);
  CHECK_HIP(hipMemcpy(f, o, nq * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(f + nq, to, nq * 4, hipMemcpyDeviceToHost));
  double num[2] = {0, 0}, den[2] = {0, 0};
  for (int t = 0; t < 2; ++t)
    for (size_t i = 0; i < nq; ++i) {
      const double a = b[t * nq + i], r = f[t * nq + i];
      num[t] += (a - r) * (a - r), den[t] += r * r;
    }
  report("bf16 and fp32 paths: status", rc == ATTN_JVP_OK && rc2 == ATTN_JVP_OK, (double)rc2);
  report("bf16 vs fp32 path: O relative Frobenius <= 1e-2", sqrt(num[0] / den[0]) <= 1e-2,
         sqrt(num[0] / den[0]));
  report("bf16 vs fp32 path: dO relative Frobenius <= 1e-2", sqrt(num[1] / den[1]) <= 1e-2,
         sqrt(num[1] / den[1]));
  for (int t = 0; t < 6; ++t) {
    CHECK_HIP(hipFree(dv[t]));
    free(h[t]);
  }
  CHECK_HIP(hipFree(o));
  CHECK_HIP(hipFree(to));
  free(f), free(b);
}

static void argument_errors(void) {
  float x = 0;
  int rc = attn_jvp_fwd(NULL, &x, &x, &x, &x, &x, &x, &x, NULL, 1, 1, 1, 1, 128, 1.0f, NULL);
  report("NULL q: EINVAL", rc == ATTN_JVP_EINVAL, (double)rc);
  rc = attn_jvp_fwd(&x, &x, &x, &x, &x, &x, &x, &x, NULL, 1, 1, 1, 1, 96, 1.0f, NULL);
  report("d = 96: EUNSUPPORTED", rc == ATTN_JVP_EUNSUPPORTED, (double)rc);
  printf("strerror(EALIGN) = %s\n", attn_jvp_strerror(ATTN_JVP_EALIGN));
}

int main(int argc, char **argv) {
  argument_errors();
  if (argc > 1 && strcmp(argv[1], "--no-gpu") == 0) {
    printf("%s\n", failures ? "FAILED" : "argument checks passed");
    return failures ? 1 : 0;
  }
  one_key();
  uniform_attention();
  bf16_vs_fp32();
  printf("%s\n", failures ? "FAILED" : "all checks passed");
  return failures ? 1 : 0;
}
