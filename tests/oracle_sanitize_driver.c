/*
 * Drives every oracle entry point once on small ragged shapes, each buffer
 * allocated at its exact size, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer reports any out-of-bounds access, use of freed
 * memory or undefined arithmetic in the oracle's C code.  Prints "ok" and a
 * checksum of the outputs.  Test infrastructure: built and run by
 * test_oracle_sanitize.py only.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "bi_oracle.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;

static double unif(void) { /* xorshift64*, uniform in [0, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t *bf16_buf(size_t n, double scale) {
  uint16_t *p = malloc(n * sizeof *p);
  for (size_t i = 0; i < n; ++i) p[i] = or_f32_to_bf16((float)((2.0 * unif() - 1.0) * scale));
  return p;
}

static uint64_t digest = 1469598103934665603ull;
static void mix(const void *p, size_t bytes) { /* FNV-1a */
  const unsigned char *c = p;
  for (size_t i = 0; i < bytes; ++i) digest = (digest ^ c[i]) * 1099511628211ull;
}

#define CHECK(call)                                      \
  do {                                                   \
    int rc_ = (call);                                    \
    if (rc_ != 0) {                                      \
      fprintf(stderr, "%s returned %d\n", #call, rc_);   \
      return 1;                                          \
    }                                                    \
  } while (0)

int main(void) {
  /* GEMM: K = 1056 is two whole 512-row segments and a 32-row tail */
  {
    const int64_t M = 3, N = 48, K = 1056;
    uint16_t *x = bf16_buf(M * K, 2.0), *w = bf16_buf(K * N, 0.1);
    uint16_t *y = malloc(M * N * sizeof *y);
    float *y32 = malloc(M * N * sizeof *y32);
    double *ye = malloc(M * N * sizeof *ye), *ya = malloc(M * N * sizeof *ya);
    CHECK(or_gemm(x, w, y, y32, M, N, K));
    CHECK(or_gemm_exact(x, w, ye, M, N, K));
    CHECK(or_gemm_absdot(x, w, ya, M, N, K));
    mix(y, M * N * sizeof *y);
    float v[3] = {1e8f, -1e8f, 1.0f};
    float f = or_fold_f32(v, 3);
    mix(&f, sizeof f);
    free(x); free(w); free(y); free(y32); free(ye); free(ya);
  }
  /* RMSNorm: H = 4104 leaves a ragged last pass of the 256-lane tree */
  {
    const int64_t M = 3, H = 4104;
    uint16_t *x = bf16_buf(M * H, 3.0), *g = bf16_buf(H, 1.0);
    uint16_t *y = malloc(M * H * sizeof *y);
    float *r = malloc(M * sizeof *r);
    double *ye = malloc(M * H * sizeof *ye);
    CHECK(or_rmsnorm(x, g, y, r, M, H, 1e-5f));
    CHECK(or_rmsnorm_exact(x, g, ye, M, H, 1e-5));
    mix(y, M * H * sizeof *y);
    free(x); free(g); free(y); free(r); free(ye);
  }
  /* Paged attention: contexts of 1, 300 and 513 tokens (chunk and page
   * edges), a shuffled page pool with no spare pages, an empty request */
  {
    const int B = 4, Hq = 8, Hkv = 2, D = 128, PS = 16;
    const int32_t ctx[4] = {1, 300, 513, 0};
    int64_t maxb = 0, P = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t nb = (ctx[b] + PS - 1) / PS;
      if (nb > maxb) maxb = nb;
      P += nb;
    }
    int32_t *bt = malloc(B * maxb * sizeof *bt);
    int32_t *perm = malloc(P * sizeof *perm);
    for (int64_t i = 0; i < P; ++i) perm[i] = (int32_t)i;
    for (int64_t i = P - 1; i > 0; --i) {
      const int64_t j = (int64_t)(unif() * (double)(i + 1));
      const int32_t t = perm[i];
      perm[i] = perm[j];
      perm[j] = t;
    }
    int64_t off = 0;
    for (int b = 0; b < B; ++b)
      for (int64_t j = 0; j < maxb; ++j)
        bt[b * maxb + j] = j < (ctx[b] + PS - 1) / PS ? perm[off++] : -1;
    uint16_t *q = bf16_buf((size_t)B * Hq * D, 1.0);
    uint16_t *kv = bf16_buf((size_t)P * 2 * Hkv * PS * D, 1.0);
    uint16_t *out = malloc((size_t)B * Hq * D * sizeof *out);
    double *oe = malloc((size_t)B * Hq * D * sizeof *oe);
    int32_t *cl = malloc(B * sizeof *cl);
    for (int b = 0; b < B; ++b) cl[b] = ctx[b];
    CHECK(or_paged_decode_attn(q, kv, bt, cl, out, B, Hq, Hkv, D, PS, maxb, 0.08838834764f));
    CHECK(or_paged_decode_attn_exact(q, kv, bt, cl, oe, B, Hq, Hkv, D, PS, maxb,
                                     0.08838834764831845));
    mix(out, (size_t)B * Hq * D * sizeof *out);
    free(bt); free(perm); free(q); free(kv); free(out); free(oe); free(cl);
  }
  /* RoPE from a row stride wider than the heads, SiLU product, add */
  {
    const int64_t M = 5, maxpos = 40, stride = 3 * 128 + 8;
    const int heads = 3, D = 128;
    float *c = malloc(maxpos * (D / 2) * sizeof *c), *s = malloc(maxpos * (D / 2) * sizeof *s);
    CHECK(or_rope_table(5e5, D, maxpos, c, s));
    uint16_t *x = bf16_buf(M * stride, 2.0);
    uint16_t *y = malloc(M * heads * D * sizeof *y);
    int32_t pos[5] = {0, 1, 17, 38, 39};
    CHECK(or_rope(x, y, pos, M, heads, D, stride, c, s, maxpos));
    int32_t past[1] = {40}; /* past the table: rejected before any access */
    if (or_rope(x, y, past, 1, heads, D, stride, c, s, maxpos) != -1) return 1;
    mix(y, M * heads * D * sizeof *y);
    const int64_t F = 40;
    uint16_t *gu = bf16_buf(M * 2 * F, 4.0), *a = malloc(M * F * sizeof *a);
    CHECK(or_silu_mul(gu, a, M, F));
    uint16_t *b = bf16_buf(M * F, 1.0), *sum = malloc(M * F * sizeof *sum);
    CHECK(or_add(a, b, sum, M * F));
    mix(sum, M * F * sizeof *sum);
    free(c); free(s); free(x); free(y); free(gu); free(a); free(b); free(sum);
  }
  /* Sampling: greedy and Gumbel rows over a vocabulary that is not a
   * multiple of the Philox block of 4 */
  {
    const int64_t M = 3, V = 1001;
    uint16_t *lg = bf16_buf(M * V, 4.0);
    uint64_t seeds[3] = {1, 2, 3}, steps[3] = {0, 5, 7};
    float temps[3] = {0.0f, 0.8f, 1.5f};
    int32_t *tok = malloc(M * sizeof *tok);
    float *best = malloc(M * sizeof *best), *second = malloc(M * sizeof *second);
    CHECK(or_sample(lg, M, V, seeds, steps, temps, tok, best, second));
    mix(tok, M * sizeof *tok);
    uint64_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, o[4];
    or_philox4x64(ctr, key, o);
    mix(o, sizeof o);
    float u = or_sample_uniform(9, 10, 1000);
    mix(&u, sizeof u);
    free(lg); free(tok); free(best); free(second);
  }
  printf("ok %016llx\n", (unsigned long long)digest);
  return 0;
}
